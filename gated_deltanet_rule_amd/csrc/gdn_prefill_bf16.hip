// gdn_prefill_bf16.hip -- chunked prefill of the gated delta rule for bf16 inputs on
// gfx950 (MI355X).
//
// Defined by: "[Model] Enable batch-invariant mixed decode and prefill for Qwen GDN",
// section "Why" (fresh prefill rows go through a 64-token chunk prefill);
// "[V1][Hybrid] GatedDeltaNet Automatic Prefix Caching", section "Purpose" (states at
// chunk boundaries returned as one flat stream); "[WIP][Kernel] Enable GDN
// batch-invariant prefix caching", section "Purpose" (one lcm(64, block) grid).
//
// Within a chunk of L <= 64 tokens (rows r, s) with start state S (d_k x d_v) the
// token recurrence S <- e^g (I - beta k k^T) S + beta k v^T is evaluated in its
// chunked form:
//     G   = inclusive cumsum of g inside the chunk,  gamma = e^G,  D[r][s] = e^(G_r - G_s)
//     A   = strictly lower part of diag(beta) (K K^T) o D
//     R   = diag(beta) (V - diag(gamma) K S)
//     U   = (I + A)^-1 R                         (a unit lower-triangular solve)
//     O   = scale (diag(gamma) Q S + (Q K^T o D o lower-incl-diagonal) U)
//     S  <- gamma_last S + K^T (diag(e^(G_last - G)) U)
//
// One workgroup owns one sequence and HG value heads that share a key head, and walks
// the sequence's chunks in order.  Per value head, d_v is split into 32-column strips
// (16-column ones when the call has no more chains than compute units), one wave
// each; a wave keeps its strip of S (d_k x 32 or d_k x 16, fp32) in MFMA accumulators
// for the whole sequence.  The d_v columns of S, R, U and O are independent, so
// strips never exchange data.  The solve runs on 16-row blocks of the chunk:
//     U_i = T_ii (R_i - sum_{j<i} A_ij U_j),   T_ii = (I + A_ii)^-1 (16 x 16)
// Per chunk, with two workgroup barriers:
//   phase 1  the first wave of each head forms its head's four diagonal K K^T tiles
//            and inverts I + A_ii by forward substitution (lane 16b + j owns column
//            j of block b); the other waves form the sixteen shared lower tiles of
//            K K^T and Q K^T (the HG heads share k and q) and turn them into the
//            -A_ij blocks and the P blocks (scale folded in) of every head.  Then,
//            per strip, Z = K S and Q S on MFMA and R = beta (V - gamma Z), V
//            entering the accumulators through an identity product from the
//            wave's own registers (each wave loads its V strip straight from HBM
//            in that operand layout, a chunk ahead)
//   stage    after the first barrier, the next chunk's prefetched Q and K rows
//            go to LDS (K and the gates by chunk parity), the first wave of each
//            head scans the next gates from its registers; the chunk after that
//            is fetched into registers once phase 3's state update is issued
//   phase 3  per strip: the block solve for U, each output row block as soon as
//            its U blocks exist, then the state update (K^T read from the K rows
//            by transposing LDS reads) and the grid export
// Precision.  Products run on the matrix cores with fp32 accumulation, in two 16-bit
// formats.  q and k are staged in LDS as fp16 (exact for the normalised keys and
// queries of the rule, down to 2^-24 below fp16's normal range), and every product
// with Q, K or K^T is an fp16 one: K K^T, Q K^T, Z = K S and Q S with S rounded once
// to fp16, and the state update with the decayed U as an fp16 hi + lo pair (x = hi +
// lo to about 2^-22).  The off-diagonal solve products -A_ij U_j take both sides as
// fp16 pairs, in three products.  The output product takes P and U as single fp16
// values, and so does T_ii X_i.  V enters exactly through a bf16 identity product.
// fp16 has four times bf16's precision, which is what lets single roundings stand
// where bf16 would need pairs; its range bounds the values: states, values and
// outputs must stay below 2^15 in magnitude.  Gates, the A_ii inverses
// and all accumulators are fp32.  A sequence's work never depends on the other
// sequences of the call, so its results are bitwise independent of its batch-mates;
// chunks lie on the absolute 64-token grid, so a resume from an exported grid state
// continues with the same arithmetic, and a partial last chunk gives its rows the
// bits the full chunk would (a row combines only rows at or before it; padding rows
// enter as exact zeros).
#include <hip/hip_runtime.h>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

using dev::kC;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- MFMA operands
//
// 16x16 output tiles: the C/D tile sits in lane l as C[4 (l / 16) + i][l % 16],
// i = 0..3.  16x16x32: lane l holds A[l % 16][k] and B[k][l % 16] for eight k; the
// "natural" order gives lane group g the k = 8g..8g+7, the "from-C" order gives it
// k = 4g..4g+3 and 16+4g..16+4g+3, the rows a pair of C tiles already holds in a
// lane.  16x16x16: lane group g holds k = 4g..4g+3, which is exactly the rows one C
// tile holds, so a C tile converted to bf16 is a B operand as it stands.

__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b),
                                                     c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32h(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16h(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// fp16 values are moved as whole 32-bit words (bit casts of packed pairs), never as
// single 16-bit lanes: this compiler merged two 16-bit stores of one pair into a
// pack of the low half twice.
__device__ __forceinline__ f16x8 cat8h(f16x4 a, f16x4 b) {
    const uint2 x = __builtin_bit_cast(uint2, a), y = __builtin_bit_cast(uint2, b);
    return __builtin_bit_cast(f16x8, make_uint4(x.x, x.y, y.x, y.y));
}

// four fp32 values rounded to fp16 (round to nearest even, two per instruction)
__device__ __forceinline__ f16x4 cvt4h(f32x4 x) {
    const f16x2 a = __builtin_convertvector((f32x2{x[0], x[1]}), f16x2);
    const f16x2 b = __builtin_convertvector((f32x2{x[2], x[3]}), f16x2);
    return __builtin_bit_cast(f16x4, make_uint2(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)));
}

// The remainder x - h of an fp32 value and an fp16 value held in the low (or high)
// half of a packed pair: one mixed-precision FMA, h (-1) + x, which is exact (the
// true result is representable) and saves widening h to fp32 first.  Probed on
// gfx950 against widening and subtracting: bitwise equal for magnitudes 2^-34 to
// 2^15, fp16 subnormals included.
__device__ __forceinline__ float rem_lo(unsigned hpair, float x) {
    float r;
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hpair), "v"(x));
    return r;
}
__device__ __forceinline__ float rem_hi(unsigned hpair, float x) {
    float r;
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hpair), "v"(x));
    return r;
}

// The lo part of x = hi + lo in fp16, given hi = x rounded to fp16: the remainder
// rounded once; x = hi + lo to about 2^-22.
__device__ __forceinline__ f16x4 lo4h(f32x4 x, f16x4 hi) {
    const uint2 w = __builtin_bit_cast(uint2, hi);
    const f16x2 a = __builtin_convertvector((f32x2{rem_lo(w.x, x[0]), rem_hi(w.x, x[1])}), f16x2);
    const f16x2 b = __builtin_convertvector((f32x2{rem_lo(w.y, x[2]), rem_hi(w.y, x[3])}), f16x2);
    return __builtin_bit_cast(f16x4, make_uint2(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)));
}

struct Split4h { f16x4 hi, lo; };
__device__ __forceinline__ Split4h split4h(f32x4 x) {
    Split4h s;
    s.hi = cvt4h(x);
    s.lo = lo4h(x, s.hi);
    return s;
}

// a bf16 pair widened and rounded to an fp16 pair (the 32-bit word in, the word out)
__device__ __forceinline__ unsigned bf16x2_to_f16x2(unsigned w) {
    const f32x2 x = {__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xffff0000u)};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(x, f16x2));
}
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 w) {
    return make_uint4(bf16x2_to_f16x2(w.x), bf16x2_to_f16x2(w.y), bf16x2_to_f16x2(w.z), bf16x2_to_f16x2(w.w));
}

__device__ __forceinline__ f16x4 ld4h(const _Float16* p) { return *reinterpret_cast<const f16x4*>(p); }
__device__ __forceinline__ f16x8 ld8h(const _Float16* p) { return *reinterpret_cast<const f16x8*>(p); }
__device__ __forceinline__ void st4h(_Float16* p, f16x4 x) { *reinterpret_cast<f16x4*>(p) = x; }

// A chunk's rows of a token-major tensor as a raw buffer: base at the chunk's first
// row (and the head's columns), nrec bytes = the chunk's valid rows.  A load at a byte
// offset at or past nrec returns zero without touching memory (the buffer's range
// check), which is how rows past a partial chunk's end enter as exact zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t rows_rsrc(const void* base, int nrec) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}
__device__ __forceinline__ uint4 ld16_rows(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float ld4_rows(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane
// 16 g + i receives element e = 0..3 from the address of lane 16 g + 4 e + i / 4, at
// position i % 4 of that lane's four values.  So if lane l points at row r0 + l / 4,
// columns c0 + 4 (l % 4) of a row-major 16-bit matrix M, lane 16 g + i gets
// M[r0 + 4 g + e][c0 + i]: the A operand of M^T (row i, k = 4 g + e) in one read.
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ f16x4 ld4_tr(const _Float16* p) {
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p)));
}

// An 8-byte LDS read the compiler keeps single.  Two 8-byte LDS reads whose addresses
// differ by a known constant are otherwise paired into one ds_read2_b64, and on gfx950
// that instruction took four times as long as the two single reads of the same bytes
// (16 cycles per wave and kilobyte against 4 to 8, in a probe that reads the Q/K row
// fragments below).  A volatile read is never paired.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) volatile u32x2 lds_vu32x2;
__device__ __forceinline__ f16x4 ld4h_single(const _Float16* p) {
    const u32x2 w = *(lds_vu32x2*)(p);
    return __builtin_bit_cast(f16x4, w);
}

// 16x32 operand of a row-major Q or K row in LDS, k from 32 ks in from-C order; sw is
// the row's column swizzle (see Smem; it only touches column bit 3)
__device__ __forceinline__ f16x8 row_fromc(const _Float16* row, int ks, int g, int sw) {
    const _Float16* p = row + ((4 * g) ^ sw);
    return cat8h(ld4h_single(p + 32 * ks), ld4h_single(p + 32 * ks + 16));
}

// B operand (from-C order, k step ks) out of a pair of state accumulator tiles, in fp16
__device__ __forceinline__ f16x8 state_frag(const f32x4& t0, const f32x4& t1) {
    return cat8h(cvt4h(t0), cvt4h(t1));
}

// Lower 16x16 blocks (i, j), j <= i, of a 64x64 matrix, numbered row by row.
__device__ __forceinline__ constexpr int blk(int i, int j) { return i * (i + 1) / 2 + j; }

// Per-token gate tables of a chunk (one head): G2 = G log2(e) (inclusive cumsum of g in
// base 2), GAM = e^G, BET = beta, KDEC = e^(G_last - G), FS = e^(G - G at the first token
// of the token's 16-row block), TE = e^(G at the last token of the block - G).  For r in
// block i and s in an earlier block j, e^(G_r - G_s) = FS_r e^(G_16i - G_16j+15) TE_s,
// three factors of at most 1.
enum { GATE_G2 = 0, GATE_GAM = 1, GATE_BET = 2, GATE_KDEC = 3, GATE_FS = 4, GATE_TE = 5, kGates = 6 };

template <int DK, int DV, int HG, int KB>
struct Smem {
    // Q and K rows (fp16).  The pitch is an odd multiple of 8 dwords and row r keeps
    // its 16-byte column groups swizzled, column c at c ^ (r & 8): with that, the
    // row-fragment reads (16 rows, one column group each), the transposing reads
    // (8 rows x 32 bytes per half wave) and the staging writes all hit distinct
    // banks.
    static constexpr int QLD = DK + 16;
    static constexpr int BLD = 24;            // rows of a 16x16 16-bit block (12 dwords:
                                              // a half wave's 8-byte row reads are
                                              // bank-conflict free)
    // block stride: 8 bf16 of padding put the four diagonal blocks (slots 0, 2, 5, 9),
    // whose columns the first wave writes in one instruction, in different banks
    static constexpr int BSZ = 16 * BLD + 8;
    static constexpr int ATLD = 20;           // rows of a transposed fp32 A_ii block
    static constexpr int ATB = 16 * ATLD + 4; // block stride (spreads the four blocks over banks)
    _Float16 q[kC * QLD];
    _Float16 k[KB][kC * QLD];                   // two: by chunk parity (the state update of
                                              // chunk c reads it while chunk c+1 is
                                              // staged); one: staged after the update
    struct Head {
        _Float16 sol[10][2][BSZ];             // block (i, j): -A_ij (j < i) as an fp16 hi,
                                              // lo pair; or T_ii, fp16, in the hi slot
        _Float16 p[10][BSZ];                  // P blocks (fp16)
        float at[4 * ATB];                    // A_ii^T: at[b * ATB + s * ATLD + r] = A_bb[r][s]
        float gate[2][kGates * kC];           // by chunk parity
    } hd[HG];
};

// Waves per SIMD the register allocation must allow: with one K buffer two workgroups
// of 32-column strips share a compute unit; a workgroup of 16-column strips has one to
// itself, two of its eight waves on each SIMD.
template <int DV, int HG, int KB, int SW>
constexpr int waves_per_simd() {
    return SW == 16 ? 2 : (HG * DV / 32) * (KB == 1 ? 2 : 1) / 4 > 1 ? (HG * DV / 32) * (KB == 1 ? 2 : 1) / 4 : 1;
}

// SW is the width of a wave's strip of value columns: 32, or 16 for calls whose
// workgroups each get a compute unit of their own (twice the waves per head, half the
// work per wave along the chain of chunks).  CS splits a head's d_v columns over that
// many workgroups (2 for calls with at most half as many chains as compute units):
// each repeats the head's shared tiles and solves its own strips, one wave per SIMD.
template <int DK, int DV, int HG, int KB, int SW, int CS>
__global__ __launch_bounds__(HG * DV / (SW * CS) * 64, (waves_per_simd<DV, HG, KB, SW>())) void chunk_kernel(PrefillArgs a) {
    using SM = Smem<DK, DV, HG, KB>;
    static_assert(CS == 1 || HG == 1, "column splits are for one head per workgroup");
    constexpr int NWH = DV / (SW * CS);      // waves per value head
    constexpr int NTL = SW / 16;             // 16-column tiles per strip
    constexpr int NW = HG * NWH;             // waves
    constexpr int NT = NW * 64;              // threads
    constexpr int MT_S = DK / 16;            // 16-row tiles of the state
    constexpr int KS_DK = DK / 32;           // 32-wide k steps over d_k
    constexpr int VPR = DK / 8;              // 16-byte vectors per Q/K row
    // Q and K rows are fetched and staged by the first head's waves alone when a
    // workgroup holds two heads of four waves: those waves win the issue arbitration
    // on their SIMDs and finish the solve first, while the other head's waves, which
    // finish it last, go straight on to it after the barrier.
    constexpr bool SPLIT = HG == 2 && NW == 8;
    constexpr int NTS = SPLIT ? NT / 2 : NT; // threads that fetch and stage Q and K
    constexpr int NQ = kC * VPR / NTS;       // prefetched Q (and K) vectors per such thread
    constexpr int NNL = HG * (NWH - 1);      // waves that are not the first of their head
    static_assert(NQ * NTS == kC * VPR, "Q/K prefetch must divide evenly");
    __shared__ __attribute__((aligned(16))) SM sm;

    const int G = a.H_v / a.H_k;
    const int GG = G / HG;
    // Workgroups go to the 8 XCDs round robin by index.  Renumber them so that each
    // XCD receives a contiguous run of (sequence, key head) units: the workgroups of
    // one sequence then share one L2, which holds the g and beta lines they all read.
    unsigned wg = blockIdx.x;
    if ((gridDim.x & 7u) == 0) wg = (wg & 7u) * (gridDim.x >> 3) + (wg >> 3);
    const int csel = (int)(wg % CS);         // this workgroup's share of the columns
    wg /= CS;
    const int seq = (int)wg / (a.H_k * GG);
    const int rem = (int)wg - seq * (a.H_k * GG);
    const int kh = rem / GG;
    const int h0 = kh * G + (rem - kh * GG) * HG;
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    int lane = tid & 63;
    const int hh = wv / NWH;                 // this wave's head within the group
    const int h = h0 + hh;
    const int col0 = SW * (wv - hh * NWH) + (DV / CS) * csel;
    // The "first" wave of each head (the one that scans the gates and inverts the
    // diagonal blocks) is wave hh of the head, so that the heads' first waves sit on
    // different SIMDs (waves go to SIMDs by index modulo 4).
    const int wi = wv - hh * NWH;            // wave index within the head
    const bool lead = wi == hh % NWH;
    typename SM::Head& hd = sm.hd[hh];

    const size_t SE = (size_t)DK * DV;
    // state strip: Sacc[mt][nt] holds S[16 mt + 4 g + i][col0 + 16 nt + li]
    f32x4 Sacc[MT_S][NTL];
    const int isl = a.init_slot ? a.init_slot[seq] : -1;
    if (isl >= 0 && isl < a.num_slots) {
        const int li = lane & 15, g4 = lane >> 4;
        const float* src = a.pool + ((size_t)isl * a.H_v + h) * SE;
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Sacc[mt][nt][i] = src[(size_t)(16 * mt + 4 * g4 + i) * DV + col0 + 16 * nt + li];
        // Wait for the state here, once: left pending, the wait would be placed at the
        // state's first use inside the chunk loop and, executed every chunk, would also
        // wait for that chunk's prefetch loads.  (s_waitcnt vmcnt(0), gfx9 encoding.)
        __builtin_amdgcn_s_waitcnt(0x0F70);
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
    // next grid point after pos0 and the number of grid states exported so far
    int64_t next_export = a.export_grid > 0 ? (pos0 / a.export_grid + 1) * a.export_grid : 0;
    int64_t exported = 0;

    const __bf16* qg = static_cast<const __bf16*>(a.q);
    const __bf16* kg = static_cast<const __bf16*>(a.k);
    const __bf16* vg = static_cast<const __bf16*>(a.v);
    __bf16* og = static_cast<__bf16*>(a.o);

    // identity B operand of the 16x16x16 product: B[4 g + e][n] = (4 g + e == n)
    bf16x4 ident;
#pragma unroll
    for (int e = 0; e < 4; ++e) ident[e] = (__bf16)((4 * (lane >> 4) + e == (lane & 15)) ? 1.f : 0.f);

    // ---- prefetch registers: Q/K row vectors, V row vectors, and (first wave of each
    //      head) this head's g and beta, one token per lane
    uint4 pq[NQ], pk[NQ];
    // this wave's V strip of a chunk in the A-operand layout of the 16x16x16 identity
    // product: pv[mt][nt] = V[16 mt + li][col0 + 16 nt + 4 g4 .. + 3]
    bf16x4 pv[4][NTL];
    float gpf = 0.f, bpf = 0.f;
    // chunk c's Q and K rows and (first wave of each head) its g and beta
    auto prefetch_qk = [&](int c, unsigned t) {
        int b0, e0;
        dev::chunk_span(c, off64, len, b0, e0);
        const int tok = lo + b0, L = e0 - b0;
        const __bf16* qb = qg + ((size_t)tok * a.H_k + kh) * DK;
        const __bf16* kb = kg + ((size_t)tok * a.H_k + kh) * DK;
        if (!SPLIT || wv < NW / 2) {
            const int nrec = L * a.H_k * DK * 2;   // the chunk's L rows
            const rsrc_t rq = rows_rsrc(qb, nrec), rk = rows_rsrc(kb, nrec);
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const unsigned i = t + NTS * j;
                const unsigned r = i / VPR, vi = i % VPR;
                const uint32_t off = (r * (unsigned)a.H_k * DK + vi * 8) * 2u;
                pq[j] = ld16_rows(rq, off);
                pk[j] = ld16_rows(rk, off);
            }
        }
        if (lead) {
            const unsigned s = t & 63;
            const uint32_t off = (s * (unsigned)a.H_v + (unsigned)h) * 4u;
            const int nrec = L * a.H_v * 4;
            gpf = ld4_rows(rows_rsrc(a.g + (size_t)tok * a.H_v, nrec), off);
            bpf = ld4_rows(rows_rsrc(a.beta + (size_t)tok * a.H_v, nrec), off);
        }
    };
    // chunk c's V strip of this wave, straight into registers (8 bytes per lane and
    // tile: 16 rows x 32 bytes per instruction)
    auto prefetch_v = [&](int c, int ln) {
        int b0, e0;
        dev::chunk_span(c, off64, len, b0, e0);
        const int tok = lo + b0, L = e0 - b0;
        const rsrc_t rv = rows_rsrc(vg + ((size_t)tok * a.H_v + h) * DV + col0, L * a.H_v * DV * 2);
        const unsigned li = (unsigned)ln & 15u, g4 = (unsigned)ln >> 4;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                const unsigned r = 16u * mt + li;
                const uint32_t off = (r * (unsigned)a.H_v * DV + 16u * nt + 4u * g4) * 2u;
                pv[mt][nt] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(rv, (int)off, 0, 0));
            }
    };
    // Write chunk c's prefetched Q rows and gates (by chunk parity) to LDS.  For chunk
    // c + 1 this runs right after the barrier that ends phase 1 of chunk c: Q was last
    // read in phase 1, and the other parity of the gates was last read in phase 3 of
    // chunk c - 1.  Doing it before phase 3 issues its stores keeps the wait for the
    // loads from waiting for those.
    auto stage_q = [&](int c, unsigned t) {
        if (!SPLIT || wv < NW / 2) {
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const unsigned i = t + NTS * j;
                const unsigned r = i / VPR, vi = i % VPR;
                const unsigned col = (vi * 8) ^ (r & 8);
                *reinterpret_cast<uint4*>(sm.q + r * SM::QLD + col) = bf16x8_to_f16x8(pq[j]);
            }
        }
        if (lead) {                          // gates of this head, lane = token
            constexpr float kLog2e = 1.4426950408889634f;
            const int ln = t & 63;
            const float G2 = dev::wave_inclusive_sum(gpf * kLog2e);
            const float G2_last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G2), kC - 1));
            // G2 at the first and the last token of this lane's 16-token block (DPP
            // row_newbcast:0 and :15; a row of 16 lanes is a block)
            const float G2_bs = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, G2), 0x150, 0xf, 0xf, false));
            const float G2_be = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, G2), 0x15f, 0xf, 0xf, false));
            float* gt = hd.gate[c & 1];
            gt[GATE_G2 * kC + ln] = G2;
            gt[GATE_GAM * kC + ln] = __builtin_amdgcn_exp2f(G2);
            gt[GATE_BET * kC + ln] = bpf;
            gt[GATE_KDEC * kC + ln] = __builtin_amdgcn_exp2f(G2_last - G2);
            gt[GATE_FS * kC + ln] = __builtin_amdgcn_exp2f(G2 - G2_bs);
            gt[GATE_TE * kC + ln] = __builtin_amdgcn_exp2f(G2_be - G2);
        }
    };
    // Chunk c's prefetched K rows: with two buffers, into the other parity at the same
    // point as Q (the state update of chunk c - 1 was its last reader); with one, after
    // the barrier that follows chunk c - 1's state update.
    auto stage_k = [&](int c, unsigned t) {
        _Float16* kb = sm.k[KB == 2 ? (c & 1) : 0];
        if (!SPLIT || wv < NW / 2) {
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const unsigned i = t + NTS * j;
                const unsigned r = i / VPR, vi = i % VPR;
                const unsigned col = (vi * 8) ^ (r & 8);
                *reinterpret_cast<uint4*>(kb + r * SM::QLD + col) = bf16x8_to_f16x8(pk[j]);
            }
        }
    };
    // Q and K loads run a chunk ahead of their staging: right after phase 1 of chunk
    // c, chunk c + 1's Q and K rows are staged; chunk c + 2's are fetched at the end of
    // chunk c's phase 3, after chunk c + 1's V strip (used in phase 1 of chunk c + 1).
    if (nchunks > 0) {
        prefetch_qk(0, (unsigned)tid);
        stage_q(0, (unsigned)tid);
        stage_k(0, (unsigned)tid);
        prefetch_v(0, lane);
        if (nchunks > 1) prefetch_qk(1, (unsigned)tid);
    }

    for (int c = 0; c < nchunks; ++c) {
        int b0, e0;
        dev::chunk_span(c, off64, len, b0, e0);
        const int tok = lo + b0, L = e0 - b0;
        const int buf = c & 1;
        // Keep lane-derived addresses inside the loop: without this the compiler hoists
        // every unrolled access's address out of the chunk loop and runs out of registers.
        int tid_l = tid;
        asm volatile("" : "+v"(lane), "+v"(tid_l));
        const int li = lane & 15, g4 = lane >> 4;
        const _Float16* kb = sm.k[KB == 2 ? buf : 0];

        dev::lds_barrier();

        // ---- phase 1.  The first wave of each head: its head's four diagonal K K^T
        //      tiles -> A_bb (fp32, in LDS only it reads), then T_bb = (I + A_bb)^-1 by
        //      forward substitution, lane 16 b + j computing column j of block b.  The
        //      other waves: the sixteen shared tiles (off-diagonal K K^T -> -A_ij, and
        //      Q K^T -> P) for every head.  Then every wave prepares its strip.
        if (lead) {
            const float* gt = hd.gate[buf];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                f16x8 kf[KS_DK];              // both operands are this block's K rows
#pragma unroll
                for (int kk = 0; kk < KS_DK; ++kk) kf[kk] = ld8h(kb + (16 * b + li) * SM::QLD + ((8 * g4) ^ (li & 8)) + 32 * kk);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KS_DK; ++kk) acc = mma32h(kf[kk], kf[kk], acc);
                const int r = 16 * b + li, s0 = 16 * b + 4 * g4;
                const float G2r = gt[GATE_G2 * kC + r];
                const float br = gt[GATE_BET * kC + r];
                const f32x4 G2s = *reinterpret_cast<const f32x4*>(gt + GATE_G2 * kC + s0);
#pragma unroll
                for (int e = 0; e < 4; ++e)   // A[r][s] at row s, column r of the transposed block
                    hd.at[b * SM::ATB + (4 * g4 + e) * SM::ATLD + li] =
                        s0 + e < r ? br * acc[e] * __builtin_amdgcn_exp2f(G2r - G2s[e]) : 0.f;
            }
            const int b = g4, jc = li;
            const float* AT = hd.at + b * SM::ATB;
            // acc starts as column jc of I: t[s] = acc[s] is then 0 above the diagonal
            // (every product added there is 0 x A), 1 on it and the substitution below
            float acc[16], t[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = r == jc ? 1.f : 0.f;
            // row s of the transposed block holds A[r][s] at column r; rows are read two
            // steps before they are used, so the LDS latency overlaps the arithmetic
            f32x4 rows[3][4];
            auto load_row = [&](int s) {
#pragma unroll
                for (int r4 = (s + 1) / 4; r4 < 4; ++r4)
                    rows[s % 3][r4] = *reinterpret_cast<const f32x4*>(AT + s * SM::ATLD + 4 * r4);
            };
            load_row(0);
            load_row(1);
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                if (s + 2 < 15) load_row(s + 2);
                t[s] = acc[s];
                if (s < 15) {
#pragma unroll
                    for (int r4 = (s + 1) / 4; r4 < 4; ++r4)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (4 * r4 + e > s) acc[4 * r4 + e] = fmaf(-rows[s % 3][r4][e], t[s], acc[4 * r4 + e]);
                }
            }
            const int bb = (0x9520 >> (4 * b)) & 15;   // blk(b, b) for b = 0..3
            unsigned short* th = reinterpret_cast<unsigned short*>(hd.sol[bb][0]);
#pragma unroll
            for (int r = 0; r < 16; r += 2) {  // rows r and r + 1 from one packed pair
                const unsigned w = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2{t[r], t[r + 1]}), f16x2));
                th[r * SM::BLD + jc] = (unsigned short)(w & 0xffffu);
                th[(r + 1) * SM::BLD + jc] = (unsigned short)(w >> 16);
            }
        } else {
            // index among the others.  Waves wv and wv ^ 4 share a SIMD (probed); with two
            // heads of four waves the first waves are 0 and 5, and their SIMD partners 4
            // and 1 take the two slots with an off-diagonal pair alone, the other four
            // waves a pair and a diagonal block each.
            const int nl = SPLIT ? (int)((0x32051040u >> (4 * wv)) & 15u)
                                 : hh * (NWH - 1) + (wi < hh % NWH ? wi : wi - 1);
            // The ten jobs, six off-diagonal block pairs (i, j) (K K^T -> -A_ij and Q K^T
            // -> P_ij, which share the K_j reads and the decay factors) and then the four
            // diagonal blocks (b, b) of Q K^T, go round robin to the NNL others: wave nl
            // takes jobs nl, nl + NNL, ...  Every wave runs the same sequence of tile
            // kinds, so the compiler can overlap them.
            const int sw = (8 * g4) ^ (li & 8);
#pragma unroll
            for (int m = 0; m < (6 + NNL - 1) / NNL; ++m) {
                const int o = nl + NNL * m;      // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
                if (o >= 6) break;
                const int i = 1 + (o >= 1) + (o >= 3), j = o - (i - 1) * i / 2;
                f16x8 fkj[KS_DK], fki[KS_DK], fqi[KS_DK];
#pragma unroll
                for (int kk = 0; kk < KS_DK; ++kk) {
                    fkj[kk] = ld8h(kb + (16 * j + li) * SM::QLD + sw + 32 * kk);
                    fki[kk] = ld8h(kb + (16 * i + li) * SM::QLD + sw + 32 * kk);
                    fqi[kk] = ld8h(sm.q + (16 * i + li) * SM::QLD + sw + 32 * kk);
                }
                f32x4 aK = {0.f, 0.f, 0.f, 0.f}, aQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KS_DK; ++kk) {
                    aK = mma32h(fkj[kk], fki[kk], aK);
                    aQ = mma32h(fkj[kk], fqi[kk], aQ);
                }
                // lane (li, g4): aX[e] = (X K^T)[r][s], r = 16 i + li, s = 16 j + 4 g4 + e
                const int r = 16 * i + li, s0 = 16 * j + 4 * g4;
#pragma unroll
                for (int x = 0; x < HG; ++x) {
                    typename SM::Head& hx = sm.hd[x];
                    const float* gx = hx.gate[buf];
                    // below the diagonal: e^(G_r - G_s) = FS_r c TE_s, c = e^(G_16i - G_16j+15)
                    const float c2 = gx[GATE_G2 * kC + 16 * i] - gx[GATE_G2 * kC + 16 * j + 15];
                    const float fr = gx[GATE_FS * kC + r] * __builtin_amdgcn_exp2f(c2);
                    const f32x4 te = *reinterpret_cast<const f32x4*>(gx + GATE_TE * kC + s0);
                    // -A_ij = -beta_r (K K^T)_rs D_rs
                    const Split4h sp = split4h(aK * te * -(fr * gx[GATE_BET * kC + r]));
                    st4h(hx.sol[blk(i, j)][0] + li * SM::BLD + 4 * g4, sp.hi);
                    st4h(hx.sol[blk(i, j)][1] + li * SM::BLD + 4 * g4, sp.lo);
                    st4h(hx.p[blk(i, j)] + li * SM::BLD + 4 * g4, cvt4h(aQ * te * (a.scale * fr)));
                }
            }
            const int b0 = (nl + 6 * NNL - 6) % NNL;   // this wave's first job past the pairs, less 6
#pragma unroll
            for (int m = 0; m < (4 + NNL - 1) / NNL; ++m) {
                const int b = b0 + NNL * m;      // a diagonal block of Q K^T: s <= r only
                if (b >= 4) break;
                f16x8 fkb[KS_DK], fqb[KS_DK];
#pragma unroll
                for (int kk = 0; kk < KS_DK; ++kk) {
                    fkb[kk] = ld8h(kb + (16 * b + li) * SM::QLD + sw + 32 * kk);
                    fqb[kk] = ld8h(sm.q + (16 * b + li) * SM::QLD + sw + 32 * kk);
                }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KS_DK; ++kk) acc = mma32h(fkb[kk], fqb[kk], acc);
                const int r = 16 * b + li, s0 = 16 * b + 4 * g4;
#pragma unroll
                for (int x = 0; x < HG; ++x) {
                    typename SM::Head& hx = sm.hd[x];
                    const float* gx = hx.gate[buf];
                    const float G2r = gx[GATE_G2 * kC + r];
                    const f32x4 G2s = *reinterpret_cast<const f32x4*>(gx + GATE_G2 * kC + s0);
                    f32x4 pd;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pd[e] = s0 + e <= r ? a.scale * acc[e] * __builtin_amdgcn_exp2f(G2r - G2s[e]) : 0.f;
                    st4h(hx.p[blk(b, b)] + li * SM::BLD + 4 * g4, cvt4h(pd));
                }
            }
        }

        // this strip's Z = K S and (Q S)^T; R = beta (V - gamma Z); S scaled by gamma_last.
        // O is accumulated transposed (value columns as rows), so that a lane ends up
        // with four consecutive columns of one output row.
        const float* gt = hd.gate[buf];
        f32x4 Racc[4][NTL], Oacc[4][NTL];
        {
            f16x8 Sb[KS_DK][NTL];
#pragma unroll
            for (int kk = 0; kk < KS_DK; ++kk)
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) Sb[kk][nt] = state_frag(Sacc[2 * kk][nt], Sacc[2 * kk + 1][nt]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) Racc[mt][nt] = Oacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KS_DK; ++kk) {
                    const f16x8 ak = row_fromc(kb + (16 * mt + li) * SM::QLD, kk, g4, li & 8);
                    const f16x8 aq = row_fromc(sm.q + (16 * mt + li) * SM::QLD, kk, g4, li & 8);
#pragma unroll
                    for (int nt = 0; nt < NTL; ++nt) {
                        Racc[mt][nt] = mma32h(ak, Sb[kk][nt], Racc[mt][nt]);
                        Oacc[mt][nt] = mma32h(Sb[kk][nt], aq, Oacc[mt][nt]);
                    }
                }
            }
        }
        const float gam_last = gt[GATE_GAM * kC + kC - 1];
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) Sacc[mt][nt] *= gam_last;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const f32x4 gam = *reinterpret_cast<const f32x4*>(gt + GATE_GAM * kC + 16 * mt + 4 * g4);
            const f32x4 bet = *reinterpret_cast<const f32x4*>(gt + GATE_BET * kC + 16 * mt + 4 * g4);
            const float sg = a.scale * gt[GATE_GAM * kC + 16 * mt + li];   // output row 16 mt + li
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                Oacc[mt][nt] *= sg;
                // + V through V I, onto -gamma Z
                Racc[mt][nt] = mma16(pv[mt][nt], ident, -gam * Racc[mt][nt]);
                Racc[mt][nt] *= bet;
            }
        }
        // chunk c + 1's V strip: this chunk's was last read just above, and issued
        // here its loads have all of phase 3 to land
        if (c + 1 < nchunks) prefetch_v(c + 1, lane);
        dev::lds_barrier();   // every -A_ij, T_ii and P block is complete
        if (c + 1 < nchunks) {
            stage_q(c + 1, (unsigned)tid_l);
            if (KB == 2) stage_k(c + 1, (unsigned)tid_l);
        }

        // ---- phase 3: U_i = T_ii (R_i - sum_{j<i} A_ij U_j); O row block i as soon as
        //      U_0..U_i exist; then the state update
        // the chunk's output rows of this strip as a raw buffer: its range check drops
        // the stores of rows past L
        const rsrc_t ro = rows_rsrc(og + ((size_t)tok * a.H_v + h) * DV + col0, L * a.H_v * DV * 2);
        const int bo = li * SM::BLD + 4 * g4;   // the lane's offset in a 16x16 block
        f16x4 Uh[4][NTL], Ul[4][NTL];             // U blocks as fp16 hi + lo pairs; hi alone in
                                              // the output product
        // X_i = R_i - sum_{j<i} A_ij U_j accumulates in Racc[i] as soon as each U_j exists
        // (right-looking), so that only one block product lies between U_i and
        // X_(i+1): block (i, j) alone on 16x16x32, A's hi and lo side by side against
        // U's hi twice, then against U's lo twice (the lo lo term comes free); blocks
        // (0, 1) of row 3 as a pair, three products (A hi U hi, A hi U lo, A lo U hi),
        // off that chain.  Every product that accumulates into X has one shape:
        // back-to-back dependent MFMAs pass the accumulator on without wait states only
        // between identical instructions, and the compiler does not pad a 16x16x32 ->
        // 16x16x16 switch on the same registers.
        auto upd1 = [&](int i, int j) __attribute__((always_inline)) {
            const f16x8 a2 = cat8h(ld4h_single(hd.sol[blk(i, j)][0] + bo), ld4h_single(hd.sol[blk(i, j)][1] + bo));
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                Racc[i][nt] = mma32h(a2, cat8h(Uh[j][nt], Uh[j][nt]), Racc[i][nt]);
                Racc[i][nt] = mma32h(a2, cat8h(Ul[j][nt], Ul[j][nt]), Racc[i][nt]);
            }
        };
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                // U_i = T_ii X_i, both single fp16 values
                const f16x4 th = ld4h_single(hd.sol[blk(i, i)][0] + bo);
                const f32x4 U = mma16h(th, cvt4h(Racc[i][nt]), f32x4{0.f, 0.f, 0.f, 0.f});
                Racc[i][nt] = U;
                Uh[i][nt] = cvt4h(U);
                Ul[i][nt] = lo4h(U, Uh[i][nt]);
            }
            if (i + 1 < 4) upd1(i + 1, i);    // the next block's last product: on the chain
            if (i == 0) upd1(2, 0);
            if (i == 1) {                     // blocks (0, 1) of row 3 as a pair
                const f16x8 ah = cat8h(ld4h_single(hd.sol[blk(3, 0)][0] + bo), ld4h_single(hd.sol[blk(3, 1)][0] + bo));
                const f16x8 al = cat8h(ld4h_single(hd.sol[blk(3, 0)][1] + bo), ld4h_single(hd.sol[blk(3, 1)][1] + bo));
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) {
                    const f16x8 uh = cat8h(Uh[0][nt], Uh[1][nt]);
                    const f16x8 ul = cat8h(Ul[0][nt], Ul[1][nt]);
                    Racc[3][nt] = mma32h(ah, uh, Racc[3][nt]);
                    Racc[3][nt] = mma32h(ah, ul, Racc[3][nt]);
                    Racc[3][nt] = mma32h(al, uh, Racc[3][nt]);
                }
            }
            // O rows 16 i .. 16 i + 15, transposed: + U_(0..i)^T P_i,(0..i)^T, U and P as
            // single fp16 values, blocks in pairs on 16x16x32 products; a last single
            // block (even i) on one 16x16x32 product too, with a zero P half (every
            // product that accumulates into O has one shape).
            const f16x4 zero4 = {};
#pragma unroll
            for (int kk = 0; 2 * kk <= i; ++kk) {
                const int j0 = 2 * kk, j1 = 2 * kk + 1;
                const f16x4 p0 = ld4h_single(hd.p[blk(i, j0)] + bo);
                const f16x8 pp = cat8h(p0, j1 <= i ? ld4h_single(hd.p[blk(i, j1)] + bo) : zero4);
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt)
                    Oacc[i][nt] = mma32h(cat8h(Uh[j0][nt], Uh[j1 <= i ? j1 : j0][nt]), pp, Oacc[i][nt]);
            }
            // Lane (li, g4) holds O[16 i + li][col0 + 16 nt + 4 g4 + e].  One row swap
            // between lane groups g4 and g4 ^ 1 (v_permlane16_swap: rows 1 and 3 of the
            // first register trade places with rows 0 and 2 of the second) leaves an
            // even group with the nt = 0 columns 4 g4 .. 4 g4 + 7 and an odd group with
            // the nt = 1 columns 12 + 4 g4 .. 12 + 4 g4 + 7: one 16-byte store per lane.
            // A 16-column strip stores its four columns per lane as they are.
            if constexpr (NTL == 1) {
                const u32x2 x = __builtin_bit_cast(u32x2, __builtin_convertvector(Oacc[i][0], bf16x4));
                const int r = 16 * i + li;
                const uint32_t off = (uint32_t)(r * a.H_v * DV + 4 * g4) * 2u;
                __builtin_amdgcn_raw_buffer_store_b64(x, ro, (int)off, 0, 0);
            } else {
                const uint2 x = __builtin_bit_cast(uint2, __builtin_convertvector(Oacc[i][0], bf16x4));
                const uint2 y = __builtin_bit_cast(uint2, __builtin_convertvector(Oacc[i][1], bf16x4));
                const auto s0 = __builtin_amdgcn_permlane16_swap(x.x, y.x, false, false);
                const auto s1 = __builtin_amdgcn_permlane16_swap(x.y, y.y, false, false);
                const u32x4 w = {s0[0], s1[0], s0[1], s1[1]};
                const int r = 16 * i + li;
                const int col = (g4 & 1) ? 12 + 4 * g4 : 4 * g4;
                const uint32_t off = (uint32_t)(r * a.H_v * DV + col) * 2u;
                __builtin_amdgcn_raw_buffer_store_b128(w, ro, (int)off, 0, 0);
            }
        }

        // S += K^T (diag(e^(G_last - G)) U), token blocks in pairs.  The B operands
        // first; then the K^T reads (transposing reads of the K rows) run two steps
        // ahead of the MFMAs that use them.
        const _Float16* ktr = kb + (lane >> 2) * SM::QLD + ((4 * (lane & 3)) ^ ((lane >> 2) & 8));
        f16x8 bh[2][NTL], bl[2][NTL];            // the decayed U as fp16 hi + lo pairs
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const f32x4 kd0 = *reinterpret_cast<const f32x4*>(gt + GATE_KDEC * kC + 32 * kk + 4 * g4);
            const f32x4 kd1 = *reinterpret_cast<const f32x4*>(gt + GATE_KDEC * kC + 32 * kk + 16 + 4 * g4);
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                const Split4h s0 = split4h(Racc[2 * kk][nt] * kd0);
                const Split4h s1 = split4h(Racc[2 * kk + 1][nt] * kd1);
                bh[kk][nt] = cat8h(s0.hi, s1.hi);
                bl[kk][nt] = cat8h(s0.lo, s1.lo);
            }
        }
        // step t = (mt, kk) = (t / 2, t % 2): K^T rows d = 16 mt + li, tokens
        // 32 kk + 4 g4 + e and 32 kk + 16 + 4 g4 + e (the from-C order)
        auto kfrag = [&](int t) {
            const int mt = t >> 1, kk = t & 1;
            const _Float16* kr = ktr + 32 * kk * SM::QLD + 16 * mt;
            return cat8h(ld4_tr(kr), ld4_tr(kr + 16 * SM::QLD));
        };
        __builtin_amdgcn_sched_barrier(0);
        {
            constexpr int NSTEP = 2 * MT_S;
            f16x8 ka[3];
            ka[0] = kfrag(0);
            ka[1] = kfrag(1);
#pragma unroll
            for (int t = 0; t < NSTEP; ++t) {
                if (t + 2 < NSTEP) ka[(t + 2) % 3] = kfrag(t + 2);
                const int mt = t >> 1, kk = t & 1;
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) {
                    Sacc[mt][nt] = mma32h(ka[t % 3], bh[kk][nt], Sacc[mt][nt]);
                    Sacc[mt][nt] = mma32h(ka[t % 3], bl[kk][nt], Sacc[mt][nt]);
                }
            }
#pragma unroll
            for (int t = 0; t < NSTEP; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * NTL, 0);   // the step's MFMAs
            }
        }
        __builtin_amdgcn_sched_barrier(0);

        // One K buffer: every wave's state update has read it once all pass the barrier.
        if (KB == 1 && c + 1 < nchunks) {
            dev::lds_barrier();
            stage_k(c + 1, (unsigned)tid_l);
        }
        // Chunk c + 2's loads go out here, after the state update: issued together with
        // the staging at the start of phase 3, their burst delayed the solve.
        if (c + 2 < nchunks) prefetch_qk(c + 2, (unsigned)tid_l);

        // ---- export on the grid
        if (a.export_grid > 0) {
            const int64_t p_end = pos0 + e0;
            if (p_end == next_export) {
                const int64_t idx = (int64_t)a.export_offsets[seq] + exported;
                next_export += a.export_grid;
                ++exported;
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

    const int fsl = a.final_slot ? a.final_slot[seq] : -1;
    if (fsl >= 0 && fsl < a.num_slots) {
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

template <int DK, int DV, int HG, int SW, int CS>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
    const int G = a.H_v / a.H_k;
    const unsigned blocks = (unsigned)a.num_seqs * (unsigned)a.H_k * (unsigned)(G / HG) * CS;
    // two K buffers, by chunk parity, spare the barrier before staging K: for the head
    // pairs and the eight 16-column waves of one head (measured: 2.8 % faster on a
    // varlen batch); one for 32-column strips, where two workgroups share a compute
    // unit, and for half heads (measured: 7.8 % faster on a mixed step than two)
    constexpr int KB = HG == 1 && (SW == 32 || CS == 2) ? 1 : 2;
    hipLaunchKernelGGL((chunk_kernel<DK, DV, HG, KB, SW, CS>), dim3(blocks), dim3(HG * DV / (SW * CS) * 64), 0, stream, a);
    return hipGetLastError();
}

template <int HG, int SW, int CS>
hipError_t launch_dims(const PrefillArgs& a, hipStream_t stream) {
    if (a.d_k == 128 && a.d_v == 128) return launch_typed<128, 128, HG, SW, CS>(a, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_typed<128, 64, HG, SW, CS>(a, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_typed<64, 128, HG, SW, CS>(a, stream);
    return launch_typed<64, 64, HG, SW, CS>(a, stream);
}

}  // namespace

// Compute units of the current device (the launch goes to it), read once per device.
int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Two value heads of a key head per workgroup share the K K^T and Q K^T tiles and
// halve the LDS traffic of staging; one head per workgroup doubles the workgroups.
// The pair is used only when it still gives every compute unit a workgroup: a call
// with few sequences (a varlen batch of a few long prompts, the prefill part of a
// mixed step) is bound by the length of its longest chain, and one head per
// workgroup runs that chain with four waves on the compute unit instead of eight.
// When even the (sequence, value head) chains do not outnumber the compute units,
// each workgroup has a compute unit to itself and its head gets eight waves of
// 16-column strips, which halves each wave's share of the chain's products; with at
// most half as many chains as compute units (and d_v = 128), a head's columns go to
// two workgroups of four such waves, one per SIMD (the shared tiles are formed in
// both).  All
// shapes run the same arithmetic per element, so a sequence's results are bitwise
// the same whichever shape its call takes.
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    const int G = a.H_v / a.H_k;
    const int64_t units = (int64_t)a.num_seqs * a.H_v;   // (sequence, value head) chains
    if (G % 2 == 0 && units / 2 >= device_cus()) return launch_dims<2, 32, 1>(a, stream);
    if (a.d_v == 128 && 2 * units <= device_cus())        // four strips per workgroup
        return a.d_k == 128 ? launch_typed<128, 128, 1, 16, 2>(a, stream) : launch_typed<64, 128, 1, 16, 2>(a, stream);
    if (units <= device_cus()) return launch_dims<1, 16, 1>(a, stream);
    return launch_dims<1, 32, 1>(a, stream);
}

}  // namespace gdn
