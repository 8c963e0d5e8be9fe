// Grouped matrix product with fp32 operands on the gfx950 bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16, sixteen times the fp32 matrix-core rate).
//
// Every fp32 operand element is split into three bf16 pieces, x = x1 + x2 + x3 with
// x1 = RN_bf16(x), x2 = RN_bf16(x - x1), x3 = x - x1 - x2.  Each bf16 holds 8
// significant bits, and after x1 the remainder has at most 16 significant bits and after
// x2 at most 8, so the three pieces represent x exactly (normal range).  The product
// x y is formed from the six partial products of order at least 2^-16 relative,
//     x1 y1 + x1 y2 + x2 y1 + x1 y3 + x3 y1 + x2 y2,
// each exact in fp32 and accumulated in fp32 by the matrix cores.  The three dropped
// products (x2 y3, x3 y2, x3 y3) are below 2^-26 |x y| with round-to-nearest pieces
// (|x2| <= 2^-9 |x|, |x3| <= 2^-17 |x|), under the 2^-24 rounding of one fp32 product, so
// the result is as accurate as the fp32 matrix-core product: the same K |a| |b| 2^-24
// error bound, a different rounding order.  Six bf16 instructions of 32 x 32 x 16 cost
// 6 / 16 of the fp32 instructions for the same 32 x 32 x 16 block.
//
// Design (large batches of large products):
//  * workgroup = 4 waves (2 x 2), each with 2 x 2 accumulator blocks of 32 x 32 (a
//    128 x 128 tile), two workgroups per CU: the two waves of a SIMD belong to different
//    workgroups, so one's split work runs beside the other's matrix-core work (larger
//    tiles with one workgroup per CU, and waves specialized into loaders and multipliers,
//    measured slower);
//  * small batches (too few 128 x 128 tiles to fill the GPU) take a 64 x 64 tile: one
//    accumulator block per wave and slices of 32 k (two matrix-core steps per slice), so
//    a workgroup still loads one run of eight k of A and one of B per thread and slice;
//  * BK = 16 (64 x 64: 32): 32 x 32 x 16 steps per slice.  Every thread loads runs of eight
//    consecutive k of rows of op(A) and op(B) per slice (two 16-byte loads where the
//    operand is K-contiguous in memory, eight 4-byte buffer loads along k where it is M- or
//    N-contiguous, each coalesced across the wave), splits them and stores each piece
//    plane as one 16-byte LDS store, K-contiguous, so every operand fragment of the matrix
//    cores is one 16-byte LDS read whatever the operand's layout in memory;
//  * LDS: for each operand and piece a [rows][BK + 8] bf16 plane (48- or 80-byte pitch:
//    consecutive rows read at distinct 16-byte bank groups), double buffered, 72 KB
//    (64 x 64: 60 KB);
//  * the split costs about 5.5 vector instructions per element loaded, against
//    TM TN 6 / (TM + TN) matrix-core instructions per element pair: large per-wave
//    tiles keep it small next to the matrix-core work;
//  * slices are loaded two ahead (two register sets).  An iteration issues the global
//    loads of slice s + 2 and the LDS fragment reads of slice s, then runs slice s's
//    matrix-core products with the split of slice s + 1 (loaded one iteration earlier)
//    interleaved between them, four vector instructions after each matrix-core one, and
//    stores the pieces last; one barrier per slice (interleaving within the wave: 3-10%
//    over splitting first and multiplying after);
//  * every load of the 16-byte path is a buffer load: rows or columns past the operand and
//    quads past K read zero from the buffer's range check, so nothing is masked (the
//    vector work per slice is the split itself: 5.5 instructions per element);
//  * the K scale of op(B)'s rows (V diag(lam) V^T) is applied to the fp32 values before
//    the split; the epilogue is the fp32 kernel's (gemm_common.hpp).
// Split-K chunks (ksplit) are supported; operands that sum split-K slabs while loading
// are not (those products take the fp32 kernel).  Operands that deny 16-byte loads (a
// caller's gradient view) are loaded four bytes at a time.
#include "gemm_common.hpp"

namespace s4 {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Tile geometry: 2 x 2 waves of TM x TN blocks of 32 x 32, slices of BK k (BK / 16
// matrix-core steps; each thread loads runs of eight k).
template <int TM_, int TN_, int BK_>
struct X3Tile {
    static constexpr int WM = 2, WN = 2, TM = TM_, TN = TN_;
    static constexpr int BM = WM * TM * 32, BN = WN * TN * 32, BK = BK_;
    static constexpr int KG = BK / 8;                     // runs of eight k per row and slice
    static constexpr int KSTEPS = BK / 16;                // 32 x 32 x 16 steps per slice
    // bf16 per LDS row: a pitch of (BK + 8) bf16 puts eight (BK = 16: 48-byte pitch) or
    // sixteen (BK = 32: 80-byte pitch) consecutive rows in distinct 16-byte bank groups
    static constexpr int PITCH = BK + 8;
    static constexpr int PLANE_A = BM * PITCH, PLANE_B = BN * PITCH;
    static constexpr int BUF = 3 * (PLANE_A + PLANE_B);   // bf16 per buffer
    static constexpr int NIA = BM * KG / 256, NIB = BN * KG / 256;   // runs per thread
    static constexpr int LDS_BYTES = 2 * BUF * 2;
    static_assert(BK == 16 || BK == 32, "slice depth");
    static_assert(BM * KG % 256 == 0 && BN * KG % 256 == 0, "whole runs per thread");
    static_assert(LDS_BYTES >= 4 * (2 * 32 * 33 + 2 * 32 * 33) && LDS_BYTES >= 4 * WM * BN,
                  "LDS too small for the epilogue");
};

// Two floats to a packed pair of bf16 (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// The three bf16 pieces of eight fp32 values, each as eight packed bf16 (k order).
__device__ __forceinline__ void split3(const float (&x)[8], u32x4& p1, u32x4& p2, u32x4& p3) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // (the empty asm keeps the compiler from re-deriving each half with a conversion
        // of its own: the pair's packed result is unpacked with one shift and one AND)
        uint32_t h = pk_bf16(x[2 * i], x[2 * i + 1]);
        asm volatile("" : "+v"(h));
        const float r0 = x[2 * i] - __uint_as_float(h << 16);
        const float r1 = x[2 * i + 1] - __uint_as_float(h & 0xffff0000u);
        uint32_t m = pk_bf16(r0, r1);
        asm volatile("" : "+v"(m));
        const float s0 = r0 - __uint_as_float(m << 16);
        const float s1 = r1 - __uint_as_float(m & 0xffff0000u);
        p1[i] = h;
        p2[i] = m;
        p3[i] = pk_bf16(s0, s1);
    }
}

// Byte offset that lies past every operand's buffer range (operands span less than 2 GiB):
// a buffer load from it returns zero.
constexpr uint32_t OUTSIDE = 0x80000000u;

// Eight consecutive k of one row of a K-contiguous operand (k along the stored row): two
// 16-byte buffer loads from byte offset off (the caller guarantees 16-byte alignment, ld %
// 4 == 0 and a K extent that is a multiple of 4, so a quad lies entirely inside or outside
// the operand).  k_ok0 / k_ok1: the quads at k and k + 4 lie before the end of K; a quad
// past it, and a row past the operand (off at or beyond OUTSIDE), reads zero.
__device__ __forceinline__ void row8(float (&v)[8], __amdgpu_buffer_rsrc_t r, uint32_t off, bool k_ok0,
                                     bool k_ok1) {
    const uint32_t q0 = k_ok0 ? off : OUTSIDE;
    const uint32_t q1 = k_ok1 ? off + 16 : OUTSIDE;
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)q0, 0, 0);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, (int)q1, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = __uint_as_float(a[e]); v[4 + e] = __uint_as_float(b[e]); }
}

// The same eight values without the 16-byte conditions: one 4-byte load each, every
// address clamped into the operand (k along the stored row when KC, else down the
// stored column c).
template <bool KC>
__device__ __forceinline__ void scalar8(float (&v)[8], const float* __restrict__ base, int64_t ld, int r, int k,
                                        int rows, int cols) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if constexpr (KC) v[e] = ldg(base + (int64_t)min(r, rows - 1) * ld + min(k + e, cols - 1));
        else v[e] = ldg(base + (int64_t)min(k + e, rows - 1) * ld + min(r, cols - 1));
    }
}

// Zeroes the out-of-range values loaded by scalar8 (row r of op(X), k..k+7 along K).
__device__ __forceinline__ void mask8(float (&v)[8], bool row_ok, int k, int K) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = keep_if(v[e], row_ok && k + e < K);
}

// Buffer resource over the `rows` stored rows of pitch ld of an operand (the last row
// counted to `cols`): a buffer load past its end returns zero, so rows past the operand
// (and k past the last stored row, down a stored column) need no mask.  The operand spans
// less than 2 GiB (checked on the host with the 16-byte-load conditions).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const float* base, int64_t ld, int rows, int cols) {
    const int bytes = (int)(((int64_t)(rows - 1) * ld + cols) * 4);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, bytes, 0x00020000);
}

// Eight consecutive k of column c of an operand stored K x cols (k along the stored
// rows): one 4-byte buffer load per k, k past the last row reads zero, and so does a
// column past the operand (off at or beyond OUTSIDE).  off: byte offset of (k, c); step:
// bytes between stored rows.
__device__ __forceinline__ void col8(float (&v)[8], __amdgpu_buffer_rsrc_t r, uint32_t off, int step) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
        v[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)(off + e * step), 0, 0));
}

// KS: op(B)'s rows are scaled by kscale[k] (the statistic V diag(lam) V^T).  VEC: every
// operand meets the 16-byte conditions and spans less than 2 GiB (else 4-byte loads with
// clamped addresses).
template <class T, bool TA, bool TB, bool KS, bool VEC>
__device__ __forceinline__ void x3_body(const GemmDesc& dsc, int t, const IoEntry* __restrict__ io,
                                        uint16_t* __restrict__ lds) {
    constexpr int WM = T::WM, TM = T::TM, TN = T::TN, BM = T::BM, BN = T::BN, BK = T::BK;
    constexpr int PITCH = T::PITCH, PLANE_A = T::PLANE_A, PLANE_B = T::PLANE_B, BUF = T::BUF;
    constexpr int NIA = T::NIA, NIB = T::NIB, KG = T::KG, KSTEPS = T::KSTEPS;
    int ks, tile_m, tile_n;
    decode_tile<BM, BN>(dsc, t, ks, tile_m, tile_n);
    const bool sym = (dsc.flags & GEMM_F_SYM) != 0;
    const bool mirror = sym && tile_m != tile_n;
    const int row0 = tile_m * BM;
    const int col0 = tile_n * BN;
    const int M = dsc.M, N = dsc.N;
    const int kbeg = ks * dsc.kchunk;
    const int K = (dsc.ksplit > 1) ? min(dsc.K, kbeg + dsc.kchunk) : dsc.K;

    const float* A = dsc.A;
    int64_t lda = dsc.lda;
    if (dsc.a_io >= 0) { A = io[dsc.a_io].G; lda = io[dsc.a_io].ldg; }
    const float* B = dsc.B;
    int64_t ldb = dsc.ldb;
    if (dsc.b_io >= 0) { B = io[dsc.b_io].G; ldb = io[dsc.b_io].ldg; }
    float* D = dsc.D + ks * dsc.dslab;
    int64_t ldd = dsc.ldd;
    if (dsc.d_io >= 0) { D = io[dsc.d_io].P; ldd = io[dsc.d_io].ldp; }
    const float* __restrict__ ksc = dsc.kscale;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int wave_m = wv % WM;
    const int wave_n = wv / WM;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    // Runs (eight k of one row) of the slice that this thread loads: item j = tid + 256 i
    // of an operand with R rows is (row (j % 8) + 8 (j / (8 KG)), run (j / 8) % KG) where
    // the operand is K-contiguous in memory (KG threads per row, 32 KG contiguous bytes;
    // eight consecutive lanes store eight rows at one run, so the 16-byte LDS stores fall
    // in distinct bank groups) and (row j % R, run j / R) where it is not (consecutive
    // rows along the wave).
    int ar[NIA], ak[NIA], br[NIB], bk[NIB];
#pragma unroll
    for (int i = 0; i < NIA; ++i) {
        const int j = tid + 256 * i;
        ar[i] = TA ? (j & (BM - 1)) : ((j & 7) + 8 * (j / (8 * KG)));
        ak[i] = TA ? (j / BM) * 8 : ((j >> 3) % KG) * 8;
    }
#pragma unroll
    for (int i = 0; i < NIB; ++i) {
        const int j = tid + 256 * i;
        br[i] = TB ? ((j & 7) + 8 * (j / (8 * KG))) : (j & (BN - 1));
        bk[i] = TB ? ((j >> 3) % KG) * 8 : (j / BN) * 8;
    }

    // VEC: every load is a buffer load over the operand as stored; a row (K-contiguous
    // operand) or column (the others) past the operand starts at OUTSIDE and reads zero,
    // and so does a quad past K, so the loaded values need no mask.  Offsets are bytes
    // from the operand's base at the thread's first slice.
    const __amdgpu_buffer_rsrc_t ra = operand_rsrc(A, lda, TA ? K : M, TA ? M : K);
    const __amdgpu_buffer_rsrc_t rb = operand_rsrc(B, ldb, TB ? N : K, TB ? K : N);
    // the K scale as a buffer of K floats: where 16-byte loads are allowed and one operand
    // is K-contiguous (so K is a multiple of 4), a run's eight scales are two 16-byte loads
    // (a quad past K reads zero); otherwise eight clamped 4-byte loads
    constexpr bool KQUAD = VEC && (!TA || TB);
    [[maybe_unused]] const __amdgpu_buffer_rsrc_t rk = operand_rsrc(KS ? ksc : A, 0, 1, K);
    const int astep = (int)(lda * 4), bstep = (int)(ldb * 4);
    uint32_t aoff[NIA], boff[NIB];
#pragma unroll
    for (int i = 0; i < NIA; ++i) {
        const int r = row0 + ar[i];
        aoff[i] = r >= M ? OUTSIDE
                : TA ? (uint32_t)(((int64_t)(kbeg + ak[i]) * lda + r) * 4)
                     : (uint32_t)(((int64_t)r * lda + kbeg + ak[i]) * 4);
    }
#pragma unroll
    for (int i = 0; i < NIB; ++i) {
        const int r = col0 + br[i];
        boff[i] = r >= N ? OUTSIDE
                : TB ? (uint32_t)(((int64_t)r * ldb + kbeg + bk[i]) * 4)
                     : (uint32_t)(((int64_t)(kbeg + bk[i]) * ldb + r) * 4);
    }

    floatx16 acc[TM][TN];
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int n = 0; n < TN; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

    struct Raw {
        float a[NIA][8], b[NIB][8], k[NIB][KS ? 8 : 1];
    };
    // slice s (k0 = kbeg + s * BK): buffer loads read zero past the operand and past K;
    // without VEC the loads are clamped and the values masked when stored
    auto load = [&](Raw& R, int s) {
        const int k0 = kbeg + s * BK;
#pragma unroll
        for (int i = 0; i < NIA; ++i) {
            if constexpr (!VEC) scalar8<!TA>(R.a[i], A, lda, row0 + ar[i], k0 + ak[i], TA ? K : M, TA ? M : K);
            else if constexpr (!TA) row8(R.a[i], ra, aoff[i] + s * BK * 4, k0 + ak[i] < K, k0 + ak[i] + 4 < K);
            else col8(R.a[i], ra, aoff[i] + s * BK * astep, astep);
        }
#pragma unroll
        for (int i = 0; i < NIB; ++i) {
            if constexpr (!VEC) scalar8<TB>(R.b[i], B, ldb, col0 + br[i], k0 + bk[i], TB ? N : K, TB ? K : N);
            else if constexpr (TB) row8(R.b[i], rb, boff[i] + s * BK * 4, k0 + bk[i] < K, k0 + bk[i] + 4 < K);
            else col8(R.b[i], rb, boff[i] + s * BK * bstep, bstep);
            if constexpr (KS && KQUAD) {
                const int kk = k0 + bk[i];
                const u32x4 qa = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(kk < K ? (uint32_t)kk * 4 : OUTSIDE), 0, 0);
                const u32x4 qb =
                    __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(kk + 4 < K ? (uint32_t)kk * 4 + 16 : OUTSIDE), 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) { R.k[i][e] = __uint_as_float(qa[e]); R.k[i][4 + e] = __uint_as_float(qb[e]); }
            } else if constexpr (KS) {
#pragma unroll
                for (int e = 0; e < 8; ++e) R.k[i][e] = ldg(ksc + min(k0 + bk[i] + e, K - 1));
            }
        }
    };

    auto store = [&](Raw& R, int buf, int s) {
        const int k0 = kbeg + s * BK;
        uint16_t* base = lds + buf * BUF;
#pragma unroll
        for (int i = 0; i < NIA; ++i) {
            if constexpr (!VEC) mask8(R.a[i], row0 + ar[i] < M, k0 + ak[i], K);
            u32x4 p1, p2, p3;
            split3(R.a[i], p1, p2, p3);
            uint16_t* pa = base + ar[i] * PITCH + ak[i];
            *reinterpret_cast<u32x4*>(pa) = p1;
            *reinterpret_cast<u32x4*>(pa + PLANE_A) = p2;
            *reinterpret_cast<u32x4*>(pa + 2 * PLANE_A) = p3;
        }
#pragma unroll
        for (int i = 0; i < NIB; ++i) {
            if constexpr (!VEC) mask8(R.b[i], col0 + br[i] < N, k0 + bk[i], K);
            if constexpr (KS) {
#pragma unroll
                for (int e = 0; e < 8; ++e) R.b[i][e] *= R.k[i][e];
            }
            u32x4 p1, p2, p3;
            split3(R.b[i], p1, p2, p3);
            uint16_t* pb = base + 3 * PLANE_A + br[i] * PITCH + bk[i];
            *reinterpret_cast<u32x4*>(pb) = p1;
            *reinterpret_cast<u32x4*>(pb + PLANE_B) = p2;
            *reinterpret_cast<u32x4*>(pb + 2 * PLANE_B) = p3;
        }
    };

    struct Frags {
        bf16x8 a[KSTEPS][3][TM], b[KSTEPS][3][TN];
    };
    auto read_frags = [&](Frags& F, int buf) {
        const uint16_t* base = lds + buf * BUF;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
            for (int p = 0; p < 3; ++p) {
#pragma unroll
                for (int m = 0; m < TM; ++m)
                    F.a[s][p][m] = *reinterpret_cast<const bf16x8*>(
                        base + p * PLANE_A + (wave_m * TM * 32 + m * 32 + l32) * PITCH + s * 16 + h * 8);
#pragma unroll
                for (int n = 0; n < TN; ++n)
                    F.b[s][p][n] = *reinterpret_cast<const bf16x8*>(
                        base + 3 * PLANE_A + p * PLANE_B + (wave_n * TN * 32 + n * 32 + l32) * PITCH + s * 16 + h * 8);
            }
    };
    // per 16-k step the six piece products in one fixed order, so every output sums its
    // terms in the same sequence whatever the tile and slice depth
    auto mfmas = [&](const Frags& F) {
        constexpr int PA[6] = {0, 0, 1, 0, 2, 1};
        constexpr int PB[6] = {0, 1, 0, 2, 0, 1};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
            for (int q = 0; q < 6; ++q)
#pragma unroll
                for (int m = 0; m < TM; ++m)
#pragma unroll
                    for (int n = 0; n < TN; ++n)
                        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.a[s][PA[q]][m], F.b[s][PB[q]][n],
                                                                            acc[m][n], 0, 0, 0);
    };

    // Two register sets: slice s + 2 is loaded while slice s is multiplied and slice s + 1
    // (loaded one iteration earlier) is split into LDS; slice s's fragments are read
    // before the split, so their LDS latency hides behind it.  Loads and stores are
    // unconditional inside the loop, so the loads stay ahead of the matrix-core work (a
    // store behind a branch pulls its loads in behind the branch); past K they read
    // zeros, and a store past K goes to the buffer read one iteration earlier, which no
    // wave reads again.
    const int nk = (K - kbeg + BK - 1) / BK;
    Raw r0, r1;
    if (nk > 0) {
        load(r0, 0);
        store(r0, 0, 0);
        load(r1, 1);
    }
    __syncthreads();
    Frags F;
    // Instruction order of an iteration: the global loads, the fragment reads, a few
    // vector instructions of the split while the fragments arrive, then each matrix-core
    // instruction followed by four of the split's vector instructions (the wave keeps its
    // own matrix core busy while it splits), the LDS stores of the split last.
    constexpr int NMFMA = 6 * T::KSTEPS * TM * TN;
    auto order = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);                // global loads
        __builtin_amdgcn_sched_group_barrier(0x100, 6 * T::KSTEPS * (TM + TN), 0);   // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);               // vector
#pragma unroll
        for (int i = 0; i < NMFMA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // matrix core
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);            // vector
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 6, 0);                // LDS stores
    };
    for (int kt = 0; kt < nk; kt += 2) {
        load(r0, kt + 2);
        read_frags(F, 0);
        store(r1, 1, kt + 1);
        mfmas(F);
        order();
        __syncthreads();
        if (kt + 1 >= nk) break;
        load(r1, kt + 3);
        read_frags(F, 1);
        store(r0, 0, kt + 2);
        mfmas(F);
        order();
        __syncthreads();
    }

    float* lds_f = reinterpret_cast<float*>(lds);
    gemm_epilogue<WM, T::WN, TM, TN>(acc, dsc, D, ldd, tile_m, row0, col0, mirror, lds_f, lds_f + 2 * 32 * 33, tid);
}

template <class T, bool TA, bool TB, bool KS, bool VEC>
__global__ __launch_bounds__(256, 2) void gemm_x3_kernel(const GemmDesc* __restrict__ descs,
                                                              const int* __restrict__ prefix, int ndesc,
                                                              const IoEntry* __restrict__ io) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::BUF];
    const int blk = gemm_block_index();
    const int item = find_item(prefix, ndesc, blk);
    x3_body<T, TA, TB, KS, VEC>(descs[item], blk - prefix[item], io, lds);
}

// Transpose mode and K scale per descriptor (uniform per workgroup).
template <class T, bool VEC>
__global__ __launch_bounds__(256, 2) void gemm_x3_kernel_mixed(const GemmDesc* __restrict__ descs,
                                                                    const int* __restrict__ prefix, int ndesc,
                                                                    const IoEntry* __restrict__ io) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::BUF];
    const int blk = gemm_block_index();
    const int item = find_item(prefix, ndesc, blk);
    const GemmDesc& d = descs[item];
    const int t = blk - prefix[item];
    if (d.kscale) {
        switch (d.flags & (GEMM_F_TA | GEMM_F_TB)) {
            case 0: x3_body<T, false, false, true, VEC>(d, t, io, lds); break;
            case GEMM_F_TB: x3_body<T, false, true, true, VEC>(d, t, io, lds); break;
            case GEMM_F_TA: x3_body<T, true, false, true, VEC>(d, t, io, lds); break;
            default: x3_body<T, true, true, true, VEC>(d, t, io, lds); break;
        }
    } else {
        switch (d.flags & (GEMM_F_TA | GEMM_F_TB)) {
            case 0: x3_body<T, false, false, false, VEC>(d, t, io, lds); break;
            case GEMM_F_TB: x3_body<T, false, true, false, VEC>(d, t, io, lds); break;
            case GEMM_F_TA: x3_body<T, true, false, false, VEC>(d, t, io, lds); break;
            default: x3_body<T, true, true, false, VEC>(d, t, io, lds); break;
        }
    }
}

// the batched tile (128 x 128, 16-k slices) and the small-batch tile (64 x 64, 32-k
// slices: the same matrix-core steps per slice and workgroup as the large tile's half)
using X3T = X3Tile<2, 2, 16>;
using X3S = X3Tile<1, 1, 32>;
static_assert(X3T::BM == GEMM_X3_BM && X3T::BN == GEMM_X3_BN, "host and kernel tile");
static_assert(X3S::BM == 64 && X3S::BN == 64, "host and kernel tile");

template <class Tile>
hipError_t launch_x3_tile(int mode, bool vec, bool kscale, const GemmDesc* descs, const int* prefix, int ndesc,
                          int ntiles, const IoEntry* io, hipStream_t stream) {
    const dim3 grid(ntiles), block(256);
#define S4_X3K(TA, TB, KS)                                                                                  \
    do {                                                                                                    \
        if (vec) S4_LAUNCH((gemm_x3_kernel<Tile, TA, TB, KS, true>), grid, block, 0, stream, descs, prefix, ndesc, io); \
        else S4_LAUNCH((gemm_x3_kernel<Tile, TA, TB, KS, false>), grid, block, 0, stream, descs, prefix, ndesc, io);    \
    } while (0)
#define S4_X3(TA, TB)                          \
    do {                                       \
        if (kscale) S4_X3K(TA, TB, true);      \
        else S4_X3K(TA, TB, false);            \
    } while (0)
    switch (mode) {
        case 0: S4_X3(false, false); break;
        case GEMM_F_TB: S4_X3(false, true); break;
        case GEMM_F_TA: S4_X3(true, false); break;
        case GEMM_F_TA | GEMM_F_TB: S4_X3(true, true); break;
        default:
            if (vec) S4_LAUNCH((gemm_x3_kernel_mixed<Tile, true>), grid, block, 0, stream, descs, prefix, ndesc, io);
            else S4_LAUNCH((gemm_x3_kernel_mixed<Tile, false>), grid, block, 0, stream, descs, prefix, ndesc, io);
            break;
    }
#undef S4_X3
#undef S4_X3K
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_x3(bool small, int mode, bool vec, bool kscale, const GemmDesc* descs, const int* prefix,
                          int ndesc, int ntiles, const IoEntry* io, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    return small ? launch_x3_tile<X3S>(mode, vec, kscale, descs, prefix, ndesc, ntiles, io, stream)
                 : launch_x3_tile<X3T>(mode, vec, kscale, descs, prefix, ndesc, ntiles, io, stream);
}

}  // namespace s4
