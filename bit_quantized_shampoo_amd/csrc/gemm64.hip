// Grouped fp64 matrix product on the gfx950 matrix cores (v_mfma_f64_16x16x4_f64), for
// the float64 statistics update ("Shampoo -- Second-Order Optimizer", "Computing the
// inverse fourth root": the root in float64, since float32 eigensolvers on a
// near-singular accumulator lose the small eigenvalues).
//
// D = alpha * op(A) op(B) + beta * C in double, op(B)'s row k scaled by kscale[k]
// (float) when set; operands are all double or all float (float operands, the caller's
// gradients, are widened as they are staged).  Workgroup = 4 waves on a 128 x 128 tile,
// each wave 64 x 64 as 4 x 4 blocks of 16 x 16 (four doubles per lane each); the K loop
// stages BK = 16 slices of op(A) and op(B) in LDS as [k][row] (double buffered, the next
// slice's global loads in flight during the current slice's matrix-core work, one barrier
// per slice).  Loads are clamped into the operand and out-of-range values zeroed with a
// bit mask; stores are predicated on the bounds.
#include "kernels.hpp"

namespace s4 {

namespace {

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int PITCH = BM + 2;            // doubles per LDS k-row (A and B alike: BM == BN)
constexpr int NLOAD = BM * BK / 256;     // elements of each operand per thread and slice

typedef double doublex4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double keep64(double v, bool keep) {
    return __longlong_as_double(__double_as_longlong(v) & (keep ? -1ll : 0ll));
}

template <class IN>
__device__ __forceinline__ double ld_el(const IN* p) {
    return (double)ldg(p);
}

// Element e (0 .. NLOAD-1) of a thread's share of one BK x 128 slice of an operand whose
// slice index runs along `fast` (the contiguous dimension in memory): thread t covers the
// 4-element runs (fast0 .. fast0 + 3) of rows `slow`, 2 runs per thread.
template <bool KFAST>
__device__ __forceinline__ void slice_coords(int t, int e, int& k, int& x) {
    const int run = t + 256 * (e >> 2), off = e & 3;
    if (KFAST) {            // memory [x][k]: runs along k (16 / 4 = 4 runs per x)
        x = run >> 2;
        k = (run & 3) * 4 + off;
    } else {                // memory [k][x]: runs along x (128 / 4 = 32 runs per k)
        k = run >> 5;
        x = (run & 31) * 4 + off;
    }
}

template <bool TA, bool TB, class IN>
__global__ __launch_bounds__(256) void gemm64_kernel(const Gemm64Desc* __restrict__ descs,
                                                     const int* __restrict__ prefix, int ndesc,
                                                     const IoEntry* __restrict__ io) {
    __shared__ double As[2][BK * PITCH];
    __shared__ double Bs[2][BK * PITCH];
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const Gemm64Desc& d = descs[item];
    const int t = blockIdx.x - prefix[item];
    const int tile_m = t % d.tiles_m, tile_n = t / d.tiles_m;
    const int row0 = tile_m * BM, col0 = tile_n * BN;
    const int M = d.M, N = d.N, K = d.K;
    const IN* __restrict__ A = reinterpret_cast<const IN*>(d.a_io >= 0 ? (const void*)io[d.a_io].G : d.A);
    const IN* __restrict__ B = reinterpret_cast<const IN*>(d.b_io >= 0 ? (const void*)io[d.b_io].G : d.B);
    const int64_t lda = d.a_io >= 0 ? io[d.a_io].ldg : d.lda;
    const int64_t ldb = d.b_io >= 0 ? io[d.b_io].ldg : d.ldb;
    const float* __restrict__ ks = d.kscale;
    const int tid = threadIdx.x;

    // op(A)[m][k]: TA -> A[k][m] (memory [k][m], runs along m), else A[m][k] (runs along k)
    // op(B)[k][n]: TB -> B[n][k] (memory [n][k], runs along k), else B[k][n] (runs along n)
    double ra[NLOAD], rb[NLOAD];
    auto load = [&](int k0) {
#pragma unroll
        for (int e = 0; e < NLOAD; ++e) {
            int k, x;
            slice_coords<!TA>(tid, e, k, x);
            const int m = row0 + x, kk = k0 + k;
            const int mc = min(m, M - 1), kc = min(kk, K - 1);
            ra[e] = ld_el(TA ? A + (int64_t)kc * lda + mc : A + (int64_t)mc * lda + kc);
        }
#pragma unroll
        for (int e = 0; e < NLOAD; ++e) {
            int k, x;
            slice_coords<TB>(tid, e, k, x);
            const int n = col0 + x, kk = k0 + k;
            const int nc = min(n, N - 1), kc = min(kk, K - 1);
            rb[e] = ld_el(TB ? B + (int64_t)nc * ldb + kc : B + (int64_t)kc * ldb + nc);
        }
    };
    auto store = [&](int buf, int k0) {
#pragma unroll
        for (int e = 0; e < NLOAD; ++e) {
            int k, x;
            slice_coords<!TA>(tid, e, k, x);
            As[buf][k * PITCH + x] = keep64(ra[e], row0 + x < M && k0 + k < K);
        }
#pragma unroll
        for (int e = 0; e < NLOAD; ++e) {
            int k, x;
            slice_coords<TB>(tid, e, k, x);
            const int kk = min(k0 + k, K - 1);
            const double s = ks ? (double)ldg(ks + kk) : 1.0;
            Bs[buf][k * PITCH + x] = keep64(rb[e] * s, col0 + x < N && k0 + k < K);
        }
    };

    const int wv = tid >> 6, lane = tid & 63;
    const int wm = (wv & 1) * 64, wn = (wv >> 1) * 64;
    const int li = lane & 15, lk = lane >> 4;
    doublex4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = doublex4{0.0, 0.0, 0.0, 0.0};

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        load(0);
        store(0, 0);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load((kt + 1) * BK);
#pragma unroll
        for (int k4 = 0; k4 < BK; k4 += 4) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[buf][(k4 + lk) * PITCH + wm + i * 16 + li];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[buf][(k4 + lk) * PITCH + wn + j * 16 + li];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store(buf ^ 1, (kt + 1) * BK);
        __syncthreads();
    }

    // epilogue: register r of a lane holds D[4 r + lk][li] of each 16 x 16 block (the
    // v_mfma_f64_16x16x4 accumulator layout, checked lane by lane on the device)
    const double alpha = d.alpha, beta = d.beta;
    const double* __restrict__ C = d.C;
    double* __restrict__ D = d.D;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = col0 + wn + j * 16 + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = row0 + wm + i * 16 + 4 * r + lk;
                if (row < M && col < N) {
                    double v = alpha * acc[i][j][r];
                    if (beta != 0.0) v = fma(beta, C[(int64_t)row * d.ldc + col], v);
                    D[(int64_t)row * d.ldd + col] = v;
                }
            }
        }
}

template <bool TA, bool TB>
hipError_t launch_mode(bool in_float, const Gemm64Desc* descs, const int* prefix, int ndesc, int ntiles,
                       const IoEntry* io, hipStream_t stream) {
    if (in_float)
        S4_LAUNCH((gemm64_kernel<TA, TB, float>), dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, io);
    else
        S4_LAUNCH((gemm64_kernel<TA, TB, double>), dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, io);
    return hipGetLastError();
}

}  // namespace

int gemm64_tiles(int M, int N) { return ((M + BM - 1) / BM) * ((N + BN - 1) / BN); }
int gemm64_tiles_m(int M) { return (M + BM - 1) / BM; }

hipError_t launch_gemm64(int mode, bool in_float, const Gemm64Desc* descs, const int* prefix, int ndesc,
                         int ntiles, const IoEntry* io, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    switch (mode) {
        case 0: return launch_mode<false, false>(in_float, descs, prefix, ndesc, ntiles, io, stream);
        case GEMM_F_TA: return launch_mode<true, false>(in_float, descs, prefix, ndesc, ntiles, io, stream);
        case GEMM_F_TB: return launch_mode<false, true>(in_float, descs, prefix, ndesc, ntiles, io, stream);
        case GEMM_F_TA | GEMM_F_TB: return launch_mode<true, true>(in_float, descs, prefix, ndesc, ntiles, io, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace s4
