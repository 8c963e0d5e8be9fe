// Grouped fp32 matrix product on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Every product of the step (Bjorck V^T V and V (V^T V), the statistics
// V diag(lam) V^T and G G^T, the power step L~ V, the Householder trailing
// updates and Q accumulation, the Rayleigh product L~ Q and the four-product
// preconditioner sandwich) goes through this kernel, batched over all blocks and
// both sides in a single launch.
//
// Design:
//  * workgroup = 4 waves (256 threads); a wave owns TM x TN blocks of 32x32
//    accumulators (16 fp32 each); the register budget is capped for two workgroups
//    per CU (two waves per SIMD hide each other's barrier and LDS waits: +20% on the
//    1024^3 products against one wave per SIMD with a few registers spilled);
//  * the K loop stages BK = 16 slices of op(A) and op(B) in LDS, double
//    buffered with a register prefetch of the next slice, one barrier per slice;
//  * LDS layout follows the global layout so that every global load is a
//    16-byte vector load and every LDS store a 16-byte store: K-contiguous
//    operands (A row-major, B transposed) are kept as [row][k] with a pitch of
//    BK+4 floats and read back with one ds_read_b128 per four k values;
//    M/N-contiguous operands (A transposed, B row-major) are kept as [k][row]
//    with a pitch of BM+8 floats and read with ds_read_b32;
//  * within an 8-wide k chunk, lane half h feeds k = 4h + s to MFMA step s,
//    a permutation of the summation order only;
//  * the epilogue applies alpha, optional row / column scales and beta * C, or
//    (COLDOT) reduces alpha * acc * C over the tile's rows into one partial row
//    per tile (used for the Rayleigh quotients q_j^T L~ q_j without writing L~ Q).
//  * a launch either has one transpose mode (specialized kernel) or mixes them
//    (one kernel, branch uniform per workgroup);
//  * split K for long-K, few-tile products: chunk s of the K range writes its own
//    partial slab and the consuming product sums the slabs while loading its
//    operand tiles (a fixed order, so results are deterministic).
#include "gemm_common.hpp"

namespace s4 {

namespace {

template <int WM, int WN, int TM, int TN>
struct Tile {
    static constexpr int BM = WM * TM * 32;
    static constexpr int BN = WN * TN * 32;
    static constexpr int BK = 16;
    static constexpr int KCP = BK + 4;
    static constexpr int AMCP = BM + 8;
    static constexpr int BMCP = BN + 8;
    static constexpr int A_KC = BM * KCP, A_MC = BK * AMCP;
    static constexpr int B_KC = BN * KCP, B_MC = BK * BMCP;
    static constexpr int A_MAX = A_KC > A_MC ? A_KC : A_MC;
    static constexpr int B_MAX = B_KC > B_MC ? B_KC : B_MC;
    static constexpr int RED = WM * BN;        // COLDOT cross-wave partials
};

// Elements (row, col..col+3) of a rows x cols operand (rows, cols >= 1) are loaded in
// two phases so that a slice's loads stay in flight across the matrix-core work of the
// previous slice: raw_quad issues the loads (addresses clamped into the operand, no
// use of the values), finish_quad later zeroes the out-of-range elements.  VEC (chosen
// per launch: 16-byte aligned base, ld and cols multiples of 4) makes a quad lie
// entirely inside or entirely outside the operand: one 16-byte load.
template <bool VEC>
__device__ __forceinline__ floatx4 raw_quad(const float* __restrict__ base, int64_t ld, int row, int col,
                                            int rows, int cols) {
    const float* p = base + (int64_t)min(row, rows - 1) * ld;
    floatx4 v;
    if constexpr (VEC) {
        v = ldg(reinterpret_cast<const floatx4*>(p + min(col, cols - 4)));
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = ldg(p + min(col + e, cols - 1));
    }
    return v;
}

template <bool VEC>
__device__ __forceinline__ floatx4 finish_quad(floatx4 v, int row, int col, int rows, int cols) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = keep_if(v[e], row < rows && (VEC ? col : col + e) < cols);
    return v;
}

// Split-K partial slabs a consuming operand sums while loading (slab order, fixed).
template <bool SLAB>
constexpr int kSlabs = SLAB ? GEMM_MAX_SLABS : 1;

// Raw loads of one quad from every slab (slab index clamped to nslab - 1).
template <bool VEC, bool SLAB>
__device__ __forceinline__ void raw_quads(floatx4 (&w)[kSlabs<SLAB>], const float* __restrict__ base,
                                          int64_t slab, int nslab, int64_t ld, int row, int col, int rows,
                                          int cols) {
#pragma unroll
    for (int s = 0; s < kSlabs<SLAB>; ++s)
        w[s] = raw_quad<VEC>(base + (int64_t)min(s, nslab - 1) * slab, ld, row, col, rows, cols);
}

template <bool VEC, bool SLAB>
__device__ __forceinline__ floatx4 finish_quads(const floatx4 (&w)[kSlabs<SLAB>], int nslab, int row, int col,
                                                int rows, int cols) {
    floatx4 v = w[0];
#pragma unroll
    for (int s = 1; s < kSlabs<SLAB>; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += keep_if(w[s][e], s < nslab);
    return finish_quad<VEC>(v, row, col, rows, cols);
}

// KW = 2: two groups of four waves split the K slices of one tile (group g takes slices
// g, g + 2, ...; the same trip count for both, a slice past K loads as zeros) and add
// their accumulators through LDS at the end: two waves per SIMD for a tile that would
// otherwise have one.  Group 0 then runs the epilogue.
template <int WM, int WN, int TM, int TN, bool TA, bool TB, bool VEC, bool SLAB, int KW = 1>
__device__ __forceinline__ void gemm_body(const GemmDesc& dsc, int t, const IoEntry* __restrict__ io,
                                          float* __restrict__ As0, float* __restrict__ Bs0) {
    using T = Tile<WM, WN, TM, TN>;
    constexpr int BM = T::BM, BN = T::BN, BK = T::BK, KCP = T::KCP, AMCP = T::AMCP, BMCP = T::BMCP;
    constexpr int A_SZ = TA ? T::A_MC : T::A_KC;
    constexpr int B_SZ = TB ? T::B_KC : T::B_MC;
    constexpr int NQA = BM * BK / 4;
    constexpr int NQB = BN * BK / 4;
    constexpr int RA = (NQA + 255) / 256;
    constexpr int RB = (NQB + 255) / 256;

    int ks, tile_m, tile_n;
    decode_tile<BM, BN>(dsc, t, ks, tile_m, tile_n);
    const bool sym = (dsc.flags & GEMM_F_SYM) != 0;
    const bool mirror = (BM == BN) && sym && tile_m != tile_n;   // square tiles only
    const int row0 = tile_m * BM;
    const int col0 = tile_n * BN;
    const int M = dsc.M, N = dsc.N;
    const int kbeg = ks * dsc.kchunk;
    const int K = (dsc.ksplit > 1) ? min(dsc.K, kbeg + dsc.kchunk) : dsc.K;   // loads stop at K

    const float* A = dsc.A;
    int64_t lda = dsc.lda;
    if (dsc.a_io >= 0) { A = io[dsc.a_io].G; lda = io[dsc.a_io].ldg; }
    const float* B = dsc.B;
    int64_t ldb = dsc.ldb;
    if (dsc.b_io >= 0) { B = io[dsc.b_io].G; ldb = io[dsc.b_io].ldg; }
    float* D = dsc.D + ks * dsc.dslab;
    int64_t ldd = dsc.ldd;
    if (dsc.d_io >= 0) { D = io[dsc.d_io].P; ldd = io[dsc.d_io].ldp; }
    const int anslab = dsc.anslab, bnslab = dsc.bnslab;
    const int64_t aslab = dsc.aslab, bslab = dsc.bslab;
    const float* __restrict__ kscale = dsc.kscale;

    const int tid = threadIdx.x & 255;
    const int kg = KW > 1 ? (int)(threadIdx.x >> 8) : 0;    // K group
    float* __restrict__ As = As0 + kg * 2 * A_SZ;
    float* __restrict__ Bs = Bs0 + kg * 2 * B_SZ;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int wave_m = wv % WM;
    const int wave_n = wv / WM;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    floatx16 acc[TM][TN];
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int n = 0; n < TN; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

    // raw operand loads of the slice in flight, and the raw K-scale values of B's rows
    struct Raw {
        floatx4 a[RA][kSlabs<SLAB>], b[RB][kSlabs<SLAB>];
        float k[RB][TB ? 4 : 1];
    };

    // The K scale (statistics: V diag(lam) V^T) is applied branch-free: without one, the
    // scale is read from B itself and replaced by 1 with a bit mask.
    const float* __restrict__ ksp = kscale ? kscale : B;
    const uint32_t ksm = kscale ? 0xffffffffu : 0u;
    auto kfac = [&](float raw) { return __uint_as_float((__float_as_uint(raw) & ksm) | (0x3f800000u & ~ksm)); };

    // quad q of a slice: (row, col) coordinates inside the operand as stored
    auto a_coord = [&](int q, int k0, int& row, int& col) {
        if constexpr (!TA) { row = row0 + q / (BK / 4); col = k0 + (q % (BK / 4)) * 4; }
        else { row = k0 + q / (BM / 4); col = row0 + (q % (BM / 4)) * 4; }
    };
    auto b_coord = [&](int q, int k0, int& row, int& col) {
        if constexpr (TB) { row = col0 + q / (BK / 4); col = k0 + (q % (BK / 4)) * 4; }
        else { row = k0 + q / (BN / 4); col = col0 + (q % (BN / 4)) * 4; }
    };

    // Every thread issues all its loads of a slice unconditionally (threads past the
    // slice's last quad reload it and do not store it), so no load sits behind a branch.
    auto load_slice = [&](Raw& R, int k0) {
#pragma unroll
        for (int r = 0; r < RA; ++r) {
            int row, col;
            a_coord(min(tid + r * 256, NQA - 1), k0, row, col);
            raw_quads<VEC, SLAB>(R.a[r], A, aslab, anslab, lda, row, col, TA ? K : M, TA ? M : K);
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            int row, col;
            b_coord(min(tid + r * 256, NQB - 1), k0, row, col);
            raw_quads<VEC, SLAB>(R.b[r], B, bslab, bnslab, ldb, row, col, TB ? N : K, TB ? K : N);
            if constexpr (TB) {
#pragma unroll
                for (int e = 0; e < 4; ++e) R.k[r][e] = ldg(ksp + min(col + e, K - 1));
            } else {
                R.k[r][0] = ldg(ksp + min(row, K - 1));
            }
        }
    };

    // masks, slab sums and the K scale are applied here, after the previous slice's
    // matrix-core work, then the slice goes to LDS
    auto store_slice = [&](const Raw& R, int buf, int k0) {
        float* as = As + buf * A_SZ;
        float* bs = Bs + buf * B_SZ;
#pragma unroll
        for (int r = 0; r < RA; ++r) {
            const int q = tid + r * 256;
            int row, col;
            a_coord(min(q, NQA - 1), k0, row, col);
            const floatx4 v = finish_quads<VEC, SLAB>(R.a[r], anslab, row, col, TA ? K : M, TA ? M : K);
            if (NQA % 256 == 0 || q < NQA) {
                if constexpr (!TA) {
                    const int i = q / (BK / 4), kq = (q % (BK / 4)) * 4;
                    *reinterpret_cast<floatx4*>(&as[i * KCP + kq]) = v;
                } else {
                    const int k = q / (BM / 4), iq = (q % (BM / 4)) * 4;
                    *reinterpret_cast<floatx4*>(&as[k * AMCP + iq]) = v;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int q = tid + r * 256;
            int row, col;
            b_coord(min(q, NQB - 1), k0, row, col);
            floatx4 v = finish_quads<VEC, SLAB>(R.b[r], bnslab, row, col, TB ? N : K, TB ? K : N);
            if constexpr (TB) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] *= kfac(R.k[r][e]);   // past K: already zero
            } else {
                const float f = kfac(R.k[r][0]);
                v[0] *= f; v[1] *= f; v[2] *= f; v[3] *= f;
            }
            if (NQB % 256 == 0 || q < NQB) {
                if constexpr (TB) {
                    const int j = q / (BK / 4), kq = (q % (BK / 4)) * 4;
                    *reinterpret_cast<floatx4*>(&bs[j * KCP + kq]) = v;
                } else {
                    const int k = q / (BN / 4), jq = (q % (BN / 4)) * 4;
                    *reinterpret_cast<floatx4*>(&bs[k * BMCP + jq]) = v;
                }
            }
        }
    };

    auto compute = [&](int cur) {
        const float* as = As + cur * A_SZ;
        const float* bs = Bs + cur * B_SZ;
#pragma unroll
        for (int kc = 0; kc < BK / 8; ++kc) {
            const int kb = kc * 8 + h * 4;
            floatx4 a[TM], b[TN];
#pragma unroll
            for (int m = 0; m < TM; ++m) {
                const int row = wave_m * TM * 32 + m * 32 + l32;
                if constexpr (!TA) {
                    a[m] = *reinterpret_cast<const floatx4*>(&as[row * KCP + kb]);
                } else {
#pragma unroll
                    for (int s = 0; s < 4; ++s) a[m][s] = as[(kb + s) * AMCP + row];
                }
            }
#pragma unroll
            for (int n = 0; n < TN; ++n) {
                const int col = wave_n * TN * 32 + n * 32 + l32;
                if constexpr (TB) {
                    b[n] = *reinterpret_cast<const floatx4*>(&bs[col * KCP + kb]);
                } else {
#pragma unroll
                    for (int s = 0; s < 4; ++s) b[n][s] = bs[(kb + s) * BMCP + col];
                }
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int m = 0; m < TM; ++m)
#pragma unroll
                    for (int n = 0; n < TN; ++n)
                        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[m][s], b[n][s],
                                                                         acc[m][n], 0, 0, 0);
        }

    };

    const int nk = ((K - kbeg + BK - 1) / BK + KW - 1) / KW;   // slices per K group
    auto kof = [&](int s) { return kbeg + (KW * s + kg) * BK; };
    Raw r0, r1;
    if (nk > 0) {
        load_slice(r0, kof(0));
        store_slice(r0, 0, kof(0));
    }
    if constexpr (TM * TN == 1 && !SLAB) {
        // Inside the loop the loads are issued unconditionally (past K they reload
        // clamped addresses and are never stored): a load behind a branch makes the wait
        // before the older set's store cover the newer set too.  With K = 0 nothing is
        // loaded (the clamps need at least one element along K).
        if (nk > 0) load_slice(r1, kof(1));
        __syncthreads();
        for (int kt = 0; kt < nk; kt += 2) {
            load_slice(r0, kof(kt + 2));
            compute(0);
            if (kt + 1 < nk) store_slice(r1, 1, kof(kt + 1));
            __syncthreads();
            if (kt + 1 >= nk) break;
            load_slice(r1, kof(kt + 3));
            compute(1);
            if (kt + 2 < nk) store_slice(r0, 0, kof(kt + 2));
            __syncthreads();
        }
    } else {
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) load_slice(r0, kof(kt + 1));
            compute(cur);
            if (more) store_slice(r0, cur ^ 1, kof(kt + 1));
            __syncthreads();
        }
    }

    if constexpr (KW > 1) {
        // group 1's accumulators through LDS (free after the loop's last barrier) into
        // group 0's, which then runs the epilogue alone (it has no workgroup barrier)
        static_assert(KW == 2, "two K groups");
        constexpr int NACC = TM * TN * 16;
        if (kg == 1) {
#pragma unroll
            for (int m = 0; m < TM; ++m)
#pragma unroll
                for (int n = 0; n < TN; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r) As0[((m * TN + n) * 16 + r) * 256 + tid] = acc[m][n][r];
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int m = 0; m < TM; ++m)
#pragma unroll
                for (int n = 0; n < TN; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[m][n][r] += As0[((m * TN + n) * 16 + r) * 256 + tid];
        }
        __syncthreads();   // the epilogue reuses the LDS
        if (kg == 1) {
            // group 0's epilogue: the column-dot form has one workgroup barrier, which
            // this group meets before leaving; the others have none
            if (dsc.flags & GEMM_F_COLDOT) __syncthreads();
            return;
        }
        (void)NACC;
    }

    gemm_epilogue<WM, WN, TM, TN>(acc, dsc, D, ldd, tile_m, row0, col0, mirror, As, Bs, tid);
}

// The mirrored-store tiles of GEMM_F_SYM: two 32 x 33 tiles in each operand buffer.
static_assert(2 * Tile<2, 2, 1, 1>::A_MC >= 2 * 32 * 33 && 2 * Tile<2, 2, 1, 1>::B_MC >= 2 * 32 * 33,
              "LDS of the 64 x 64 tile too small for the mirrored stores");
static_assert(2 * Tile<2, 2, 2, 2>::A_MC >= 2 * 32 * 33 && 2 * Tile<2, 2, 2, 2>::B_MC >= 2 * 32 * 33,
              "LDS of the 128 x 128 tile too small for the mirrored stores");

// One transpose mode for the whole launch, 16-byte loads, no split-K slabs.
template <int WM, int WN, int TM, int TN, bool TA, bool TB, int KW>
__global__ __launch_bounds__(256 * KW, 2) void gemm_kernel(const GemmDesc* __restrict__ descs,
                                                        const int* __restrict__ prefix, int ndesc,
                                                        const IoEntry* __restrict__ io) {
    using T = Tile<WM, WN, TM, TN>;
    constexpr int A_SZ = TA ? T::A_MC : T::A_KC;
    constexpr int B_SZ = TB ? T::B_KC : T::B_MC;
    constexpr int A_NEED = (KW > 1 && TM * TN * 16 * 256 > T::RED) ? TM * TN * 16 * 256 : T::RED;
    constexpr int A_ALL = (2 * KW * A_SZ > A_NEED) ? 2 * KW * A_SZ : A_NEED;
    __shared__ __attribute__((aligned(16))) float As[A_ALL];
    __shared__ __attribute__((aligned(16))) float Bs[2 * KW * B_SZ];
    const int blk = gemm_block_index();
    const int item = find_item(prefix, ndesc, blk);
    gemm_body<WM, WN, TM, TN, TA, TB, true, false, KW>(descs[item], blk - prefix[item], io, As, Bs);
}

// Transpose mode per descriptor (uniform per workgroup); VEC and SLAB per launch.
template <int WM, int WN, int TM, int TN, bool VEC, bool SLAB, int KW>
__global__ __launch_bounds__(256 * KW, 2) void gemm_kernel_mixed(const GemmDesc* __restrict__ descs,
                                                              const int* __restrict__ prefix, int ndesc,
                                                              const IoEntry* __restrict__ io) {
    using T = Tile<WM, WN, TM, TN>;
    constexpr int A_NEED = (KW > 1 && TM * TN * 16 * 256 > T::RED) ? TM * TN * 16 * 256 : T::RED;
    constexpr int A_ALL = (2 * KW * T::A_MAX > A_NEED) ? 2 * KW * T::A_MAX : A_NEED;
    __shared__ __attribute__((aligned(16))) float As[A_ALL];
    __shared__ __attribute__((aligned(16))) float Bs[2 * KW * T::B_MAX];
    const int blk = gemm_block_index();
    const int item = find_item(prefix, ndesc, blk);
    const GemmDesc& d = descs[item];
    const int t = blk - prefix[item];
    switch (d.flags & (GEMM_F_TA | GEMM_F_TB)) {
        case 0: gemm_body<WM, WN, TM, TN, false, false, VEC, SLAB, KW>(d, t, io, As, Bs); break;
        case GEMM_F_TB: gemm_body<WM, WN, TM, TN, false, true, VEC, SLAB, KW>(d, t, io, As, Bs); break;
        case GEMM_F_TA: gemm_body<WM, WN, TM, TN, true, false, VEC, SLAB, KW>(d, t, io, As, Bs); break;
        default: gemm_body<WM, WN, TM, TN, true, true, VEC, SLAB, KW>(d, t, io, As, Bs); break;
    }
}

template <int WM, int WN, int TM, int TN, int KW = 1>
hipError_t launch_cfg(int mode, bool vec, bool slab, const GemmDesc* descs, const int* prefix, int ndesc,
                      int ntiles, const IoEntry* io, hipStream_t stream) {
    dim3 grid(ntiles), block(256 * KW);
    if constexpr (KW > 1) {   // K groups: 16-byte loads without split-K slabs only
        if (!vec || slab) return hipErrorInvalidValue;
        if (mode == GEMM_MODE_MIXED)
            S4_LAUNCH((gemm_kernel_mixed<WM, WN, TM, TN, true, false, KW>), grid, block, 0, stream, descs, prefix, ndesc, io);
        else if (mode == 0)
            S4_LAUNCH((gemm_kernel<WM, WN, TM, TN, false, false, KW>), grid, block, 0, stream, descs, prefix, ndesc, io);
        else if (mode == GEMM_F_TB)
            S4_LAUNCH((gemm_kernel<WM, WN, TM, TN, false, true, KW>), grid, block, 0, stream, descs, prefix, ndesc, io);
        else if (mode == GEMM_F_TA)
            S4_LAUNCH((gemm_kernel<WM, WN, TM, TN, true, false, KW>), grid, block, 0, stream, descs, prefix, ndesc, io);
        else
            S4_LAUNCH((gemm_kernel<WM, WN, TM, TN, true, true, KW>), grid, block, 0, stream, descs, prefix, ndesc, io);
        return hipGetLastError();
    }
    if (!vec || slab || mode == GEMM_MODE_MIXED) {
        if (vec && slab)
            S4_LAUNCH((gemm_kernel_mixed<WM, WN, TM, TN, true, true, 1>), grid, block, 0, stream, descs, prefix, ndesc, io);
        else if (vec)
            S4_LAUNCH((gemm_kernel_mixed<WM, WN, TM, TN, true, false, 1>), grid, block, 0, stream, descs, prefix, ndesc, io);
        else if (slab)
            S4_LAUNCH((gemm_kernel_mixed<WM, WN, TM, TN, false, true, 1>), grid, block, 0, stream, descs, prefix, ndesc, io);
        else
            S4_LAUNCH((gemm_kernel_mixed<WM, WN, TM, TN, false, false, 1>), grid, block, 0, stream, descs, prefix, ndesc, io);
        return hipGetLastError();
    }
    switch (mode) {
        case 0:
            S4_LAUNCH((gemm_kernel<WM, WN, TM, TN, false, false, 1>), grid, block, 0, stream, descs, prefix, ndesc, io);
            break;
        case GEMM_F_TB:
            S4_LAUNCH((gemm_kernel<WM, WN, TM, TN, false, true, 1>), grid, block, 0, stream, descs, prefix, ndesc, io);
            break;
        case GEMM_F_TA:
            S4_LAUNCH((gemm_kernel<WM, WN, TM, TN, true, false, 1>), grid, block, 0, stream, descs, prefix, ndesc, io);
            break;
        default:
            S4_LAUNCH((gemm_kernel<WM, WN, TM, TN, true, true, 1>), grid, block, 0, stream, descs, prefix, ndesc, io);
            break;
    }
    return hipGetLastError();
}

}  // namespace

bool gemm_vec_ok(const GemmDesc& d) {
    const bool ta = d.flags & GEMM_F_TA, tb = d.flags & GEMM_F_TB;
    // (the bf16 split kernel also needs each operand to span less than 2 GiB: its buffer
    // loads take 32-bit offsets)
    auto ok = [](const void* p, int64_t ld, int64_t rows, int64_t extent, int nslab, int64_t slab) {
        return (reinterpret_cast<uintptr_t>(p) & 15) == 0 && (ld & 3) == 0 && (extent & 3) == 0 &&
               (nslab <= 1 || (slab & 3) == 0) && (rows - 1) * ld + extent < (int64_t(1) << 29);
    };
    const int64_t ea = ta ? d.M : d.K, eb = tb ? d.K : d.N;
    const int64_t ra = ta ? d.K : d.M, rb = tb ? d.N : d.K;
    const bool a = d.a_io >= 0 ? (ea & 3) == 0 : ok(d.A, d.lda, ra, ea, d.anslab, d.aslab);
    const bool b = d.b_io >= 0 ? (eb & 3) == 0 : ok(d.B, d.ldb, rb, eb, d.bnslab, d.bslab);
    return a && b;
}

void gemm_tile_dims(int cfg, int* bm, int* bn) {
    switch (cfg) {
        case GEMM_128x128: *bm = 128; *bn = 128; break;
        case GEMM_X3: *bm = GEMM_X3_BM; *bn = GEMM_X3_BN; break;
        case GEMM_X3_64:
        case GEMM_64x64:
        case GEMM_64x64_K2: *bm = 64; *bn = 64; break;
        case GEMM_128x32: *bm = 128; *bn = 32; break;
        default: *bm = 32; *bn = 128; break;
    }
}

hipError_t launch_gemm(int cfg, int mode, bool vec, bool slab, bool kscale, const GemmDesc* descs,
                       const int* prefix, int ndesc, int ntiles, const IoEntry* io, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    switch (cfg) {
        case GEMM_128x128: return launch_cfg<2, 2, 2, 2>(mode, vec, slab, descs, prefix, ndesc, ntiles, io, stream);
        case GEMM_X3:
        case GEMM_X3_64:
            if (slab) return hipErrorInvalidValue;
            return launch_gemm_x3(cfg == GEMM_X3_64, mode, vec, kscale, descs, prefix, ndesc, ntiles, io, stream);
        case GEMM_64x64: return launch_cfg<2, 2, 1, 1>(mode, vec, slab, descs, prefix, ndesc, ntiles, io, stream);
        case GEMM_64x64_K2:   // (the K groups need 16-byte loads: a per-call caller operand may deny them)
            if (!vec || slab) return launch_cfg<2, 2, 1, 1>(mode, vec, slab, descs, prefix, ndesc, ntiles, io, stream);
            return launch_cfg<2, 2, 1, 1, 2>(mode, vec, slab, descs, prefix, ndesc, ntiles, io, stream);
        case GEMM_128x32: return launch_cfg<4, 1, 1, 1>(mode, vec, slab, descs, prefix, ndesc, ntiles, io, stream);
        default: return launch_cfg<1, 4, 1, 1>(mode, vec, slab, descs, prefix, ndesc, ntiles, io, stream);
    }
}

}  // namespace s4
