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
//    accumulators (16 fp32 each);
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
#include "kernels.hpp"

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

__device__ __forceinline__ floatx4 load_quad(const float* __restrict__ base, int64_t ld,
                                             int row, int col, int rows, int cols, bool vec_ok);

// Sum of `nslab` split-K partials (slab stride `slab` elements); one slab is a plain load.
__device__ __forceinline__ floatx4 load_quad_sum(const float* __restrict__ base, int64_t slab, int nslab,
                                                 int64_t ld, int row, int col, int rows, int cols,
                                                 bool vec_ok) {
    floatx4 v = load_quad(base, ld, row, col, rows, cols, vec_ok);
    for (int s = 1; s < nslab; ++s) {
        const floatx4 w = load_quad(base + s * slab, ld, row, col, rows, cols, vec_ok);
        v[0] += w[0]; v[1] += w[1]; v[2] += w[2]; v[3] += w[3];
    }
    return v;
}

__device__ __forceinline__ floatx4 load_quad(const float* __restrict__ base, int64_t ld,
                                             int row, int col, int rows, int cols, bool vec_ok) {
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (row >= rows) return v;
    const float* p = base + (int64_t)row * ld + col;
    if (vec_ok && col + 3 < cols) {
        v = *reinterpret_cast<const floatx4*>(p);
    } else {
        if (col + 0 < cols) v[0] = p[0];
        if (col + 1 < cols) v[1] = p[1];
        if (col + 2 < cols) v[2] = p[2];
        if (col + 3 < cols) v[3] = p[3];
    }
    return v;
}

template <int WM, int WN, int TM, int TN, bool TA, bool TB>
__device__ __forceinline__ void gemm_body(const GemmDesc& dsc, int t, const IoEntry* __restrict__ io,
                                          float* __restrict__ As, float* __restrict__ Bs) {
    using T = Tile<WM, WN, TM, TN>;
    constexpr int BM = T::BM, BN = T::BN, BK = T::BK, KCP = T::KCP, AMCP = T::AMCP, BMCP = T::BMCP;
    constexpr int A_SZ = TA ? T::A_MC : T::A_KC;
    constexpr int B_SZ = TB ? T::B_KC : T::B_MC;
    constexpr int NQA = BM * BK / 4;
    constexpr int NQB = BN * BK / 4;
    constexpr int RA = (NQA + 255) / 256;
    constexpr int RB = (NQB + 255) / 256;

    const int tiles_m = dsc.tiles_m;
    const int tiles_mn = tiles_m * ((dsc.N + BN - 1) / BN);
    const int ks = t / tiles_mn;                 // split-K chunk (0 without split)
    const int tmn = t - ks * tiles_mn;
    const int tile_m = tmn % tiles_m;
    const int row0 = tile_m * BM;
    const int col0 = (tmn / tiles_m) * BN;
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

    const bool avec = ((reinterpret_cast<uintptr_t>(A) & 15) == 0) && ((lda & 3) == 0);
    const bool bvec = ((reinterpret_cast<uintptr_t>(B) & 15) == 0) && ((ldb & 3) == 0);

    const int tid = threadIdx.x;
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

    floatx4 ra[RA], rb[RB];

    auto load_slice = [&](int k0) {
#pragma unroll
        for (int r = 0; r < RA; ++r) {
            const int q = tid + r * 256;
            if (q < NQA) {
                if constexpr (!TA) {
                    const int i = q / (BK / 4), kq = (q % (BK / 4)) * 4;
                    ra[r] = load_quad_sum(A, aslab, anslab, lda, row0 + i, k0 + kq, M, K, avec);
                } else {
                    const int k = q / (BM / 4), iq = (q % (BM / 4)) * 4;
                    ra[r] = load_quad_sum(A, aslab, anslab, lda, k0 + k, row0 + iq, K, M, avec);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int q = tid + r * 256;
            if (q < NQB) {
                if constexpr (TB) {
                    const int j = q / (BK / 4), kq = (q % (BK / 4)) * 4;
                    floatx4 v = load_quad_sum(B, bslab, bnslab, ldb, col0 + j, k0 + kq, N, K, bvec);
                    if (kscale) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (k0 + kq + e < K) v[e] *= kscale[k0 + kq + e];
                    }
                    rb[r] = v;
                } else {
                    const int k = q / (BN / 4), jq = (q % (BN / 4)) * 4;
                    floatx4 v = load_quad_sum(B, bslab, bnslab, ldb, k0 + k, col0 + jq, K, N, bvec);
                    if (kscale && k0 + k < K) {
                        const float s = kscale[k0 + k];
                        v[0] *= s; v[1] *= s; v[2] *= s; v[3] *= s;
                    }
                    rb[r] = v;
                }
            }
        }
    };

    auto store_slice = [&](int buf) {
        float* as = As + buf * A_SZ;
        float* bs = Bs + buf * B_SZ;
#pragma unroll
        for (int r = 0; r < RA; ++r) {
            const int q = tid + r * 256;
            if (q < NQA) {
                if constexpr (!TA) {
                    const int i = q / (BK / 4), kq = (q % (BK / 4)) * 4;
                    *reinterpret_cast<floatx4*>(&as[i * KCP + kq]) = ra[r];
                } else {
                    const int k = q / (BM / 4), iq = (q % (BM / 4)) * 4;
                    *reinterpret_cast<floatx4*>(&as[k * AMCP + iq]) = ra[r];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int q = tid + r * 256;
            if (q < NQB) {
                if constexpr (TB) {
                    const int j = q / (BK / 4), kq = (q % (BK / 4)) * 4;
                    *reinterpret_cast<floatx4*>(&bs[j * KCP + kq]) = rb[r];
                } else {
                    const int k = q / (BN / 4), jq = (q % (BN / 4)) * 4;
                    *reinterpret_cast<floatx4*>(&bs[k * BMCP + jq]) = rb[r];
                }
            }
        }
    };

    const int nk = (K - kbeg + BK - 1) / BK;
    if (nk > 0) {
        load_slice(kbeg);
        store_slice(0);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) load_slice(kbeg + (kt + 1) * BK);
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

        if (more) store_slice(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator register r of lane (h, l32) holds
    // row 8*(r/4) + 4*h + (r%4), column l32 of its 32x32 block.
    const float alpha = dsc.alpha, beta = dsc.beta;
    const float* __restrict__ C = dsc.C;
    const int64_t ldc = dsc.ldc;

    if (dsc.flags & GEMM_F_COLDOT) {
        // LDS is free after the final barrier of the K loop: reuse As for partials
        float* red = As;
#pragma unroll
        for (int n = 0; n < TN; ++n) {
            const int lcol = wave_n * TN * 32 + n * 32 + l32;
            const int col = col0 + lcol;
            float s = 0.f;
            if (col < N) {
#pragma unroll
                for (int m = 0; m < TM; ++m)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = row0 + wave_m * TM * 32 + m * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
                        if (row < M) s += acc[m][n][r] * C[(int64_t)row * ldc + col];
                    }
            }
            s += __shfl_xor(s, 32);
            if (h == 0) red[wave_m * BN + lcol] = s;
        }
        __syncthreads();
        if (wave_m == 0 && h == 0) {
#pragma unroll
            for (int n = 0; n < TN; ++n) {
                const int lcol = wave_n * TN * 32 + n * 32 + l32;
                const int col = col0 + lcol;
                float s = 0.f;
#pragma unroll
                for (int w = 0; w < WM; ++w) s += red[w * BN + lcol];
                if (col < N) D[(int64_t)tile_m * ldd + col] = alpha * s;
            }
        }
        return;
    }

    const float* __restrict__ rs = dsc.rscale;
    const float* __restrict__ cs = dsc.cscale;
#pragma unroll
    for (int n = 0; n < TN; ++n) {
        const int col = col0 + wave_n * TN * 32 + n * 32 + l32;
        if (col >= N) continue;
        const float csv = cs ? cs[col] : 1.f;
#pragma unroll
        for (int m = 0; m < TM; ++m) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + wave_m * TM * 32 + m * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
                if (row < M) {
                    float v = alpha * acc[m][n][r];
                    if (rs) v *= rs[row];
                    v *= csv;
                    if (beta != 0.f) v += beta * C[(int64_t)row * ldc + col];
                    D[(int64_t)row * ldd + col] = v;
                }
            }
        }
    }
}

template <int WM, int WN, int TM, int TN, bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmDesc* __restrict__ descs,
                                                   const int* __restrict__ prefix, int ndesc,
                                                   const IoEntry* __restrict__ io) {
    using T = Tile<WM, WN, TM, TN>;
    constexpr int A_SZ = TA ? T::A_MC : T::A_KC;
    constexpr int B_SZ = TB ? T::B_KC : T::B_MC;
    constexpr int A_ALL = (2 * A_SZ > T::RED) ? 2 * A_SZ : T::RED;
    __shared__ __attribute__((aligned(16))) float As[A_ALL];
    __shared__ __attribute__((aligned(16))) float Bs[2 * B_SZ];
    const int item = find_item(prefix, ndesc, blockIdx.x);
    gemm_body<WM, WN, TM, TN, TA, TB>(descs[item], blockIdx.x - prefix[item], io, As, Bs);
}

template <int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(256) void gemm_kernel_mixed(const GemmDesc* __restrict__ descs,
                                                         const int* __restrict__ prefix, int ndesc,
                                                         const IoEntry* __restrict__ io) {
    using T = Tile<WM, WN, TM, TN>;
    constexpr int A_ALL = (2 * T::A_MAX > T::RED) ? 2 * T::A_MAX : T::RED;
    __shared__ __attribute__((aligned(16))) float As[A_ALL];
    __shared__ __attribute__((aligned(16))) float Bs[2 * T::B_MAX];
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const GemmDesc& d = descs[item];
    const int t = blockIdx.x - prefix[item];
    switch (d.flags & (GEMM_F_TA | GEMM_F_TB)) {
        case 0: gemm_body<WM, WN, TM, TN, false, false>(d, t, io, As, Bs); break;
        case GEMM_F_TB: gemm_body<WM, WN, TM, TN, false, true>(d, t, io, As, Bs); break;
        case GEMM_F_TA: gemm_body<WM, WN, TM, TN, true, false>(d, t, io, As, Bs); break;
        default: gemm_body<WM, WN, TM, TN, true, true>(d, t, io, As, Bs); break;
    }
}

template <int WM, int WN, int TM, int TN>
hipError_t launch_cfg(int mode, const GemmDesc* descs, const int* prefix, int ndesc, int ntiles,
                      const IoEntry* io, hipStream_t stream) {
    dim3 grid(ntiles), block(256);
    switch (mode) {
        case 0:
            S4_LAUNCH((gemm_kernel<WM, WN, TM, TN, false, false>), grid, block, 0, stream,
                               descs, prefix, ndesc, io);
            break;
        case GEMM_F_TB:
            S4_LAUNCH((gemm_kernel<WM, WN, TM, TN, false, true>), grid, block, 0, stream,
                               descs, prefix, ndesc, io);
            break;
        case GEMM_F_TA:
            S4_LAUNCH((gemm_kernel<WM, WN, TM, TN, true, false>), grid, block, 0, stream,
                               descs, prefix, ndesc, io);
            break;
        case GEMM_F_TA | GEMM_F_TB:
            S4_LAUNCH((gemm_kernel<WM, WN, TM, TN, true, true>), grid, block, 0, stream,
                               descs, prefix, ndesc, io);
            break;
        default:
            S4_LAUNCH((gemm_kernel_mixed<WM, WN, TM, TN>), grid, block, 0, stream, descs,
                               prefix, ndesc, io);
            break;
    }
    return hipGetLastError();
}

}  // namespace

void gemm_tile_dims(int cfg, int* bm, int* bn) {
    switch (cfg) {
        case GEMM_128x128: *bm = 128; *bn = 128; break;
        case GEMM_64x64: *bm = 64; *bn = 64; break;
        default: *bm = 32; *bn = 128; break;
    }
}

hipError_t launch_gemm(int cfg, int mode, const GemmDesc* descs, const int* prefix, int ndesc, int ntiles,
                       const IoEntry* io, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    switch (cfg) {
        case GEMM_128x128: return launch_cfg<2, 2, 2, 2>(mode, descs, prefix, ndesc, ntiles, io, stream);
        case GEMM_64x64: return launch_cfg<2, 2, 1, 1>(mode, descs, prefix, ndesc, ntiles, io, stream);
        default: return launch_cfg<1, 4, 1, 1>(mode, descs, prefix, ndesc, ntiles, io, stream);
    }
}

}  // namespace s4
