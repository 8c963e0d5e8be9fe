// Diagonal fallback of a block side ("Shampoo -- Second-Order Optimizer", "Blocked and
// distributed variants": a side whose dimension exceeds a threshold drops its factor and
// keeps diagonal AdaGrad along it).  Such a side keeps only the diagonal of its factor as
// the same exponential moving average, lam_i <- beta lam_i + (1 - beta) sum_j Gs[i][j]^2
// (Gs = G for side L, G^T for side R), and its root is diag((lam + eps)^(-1/4)).
//  * diag_partials: per tile of DIAG_TR rows x DIAG_TC columns of G, the partial row sums
//                   and column sums of G^2 into workspace slabs (one read of G; columns
//                   summed down the rows in order, rows summed by a fixed butterfly);
//  * diag_ema:      lam_j <- beta lam_j + (1 - beta) sum_t slab[t][j] (slabs in order);
//  * diag_scale:    P = diag(d_L) G diag(d_R) for blocks with both sides diagonal.
// All three are bandwidth-bound streams over G (and P).
#include "kernels.hpp"

namespace s4 {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
    // butterfly over the 64 lanes: every lane ends with the same sum, in a fixed order
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__global__ __launch_bounds__(256) void diag_partials_kernel(const DiagDesc* __restrict__ descs,
                                                            const int* __restrict__ prefix, int ndesc,
                                                            const IoEntry* __restrict__ io) {
    __shared__ float wsum[4][DIAG_TR];
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const DiagDesc& d = descs[item];
    const int t = blockIdx.x - prefix[item];
    const int tm = t / d.tiles_n, tn = t - tm * d.tiles_n;
    const int r0 = tm * DIAG_TR;
    const int c = tn * DIAG_TC + (int)threadIdx.x;
    const float* __restrict__ G = io[d.blk].G;
    const int64_t ld = io[d.blk].ldg;
    const int cc = min(c, d.n - 1);
    const uint32_t cmask = c < d.n ? 0xffffffffu : 0u;
    // every row's load (clamped address) before any use; out-of-range values masked to 0
    float v[DIAG_TR];
#pragma unroll
    for (int r = 0; r < DIAG_TR; ++r) v[r] = ldg(G + (int64_t)min(r0 + r, d.m - 1) * ld + cc);
    float colsum = 0.f;
#pragma unroll
    for (int r = 0; r < DIAG_TR; ++r) {
        const uint32_t m = (r0 + r < d.m) ? cmask : 0u;
        const float x = __uint_as_float(__float_as_uint(v[r]) & m);
        v[r] = x * x;
        colsum += v[r];
    }
    if (d.colpart && c < d.n) stg(d.colpart + (int64_t)tm * d.n + c, colsum);
    if (d.rowpart) {
        const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
        for (int r = 0; r < DIAG_TR; ++r) {
            const float s = wave_sum(v[r]);
            if (lane == 0) wsum[wv][r] = s;
        }
        __syncthreads();
        const int r = threadIdx.x;
        if (r < DIAG_TR && r0 + r < d.m)
            stg(d.rowpart + (int64_t)tn * d.m + r0 + r, ((wsum[0][r] + wsum[1][r]) + wsum[2][r]) + wsum[3][r]);
    }
}

// lam_j = beta lam_j + (1 - beta) sum_{t < rows} a[t * ld + j]; non-finite raises the flag
__global__ __launch_bounds__(256) void diag_ema_kernel(const VecDesc* __restrict__ descs,
                                                       const int* __restrict__ prefix, int ndesc, float beta,
                                                       uint32_t* __restrict__ flag) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const VecDesc& d = descs[item];
    const int j = (blockIdx.x - prefix[item]) * 256 + threadIdx.x;
    if (j >= d.p) return;
    float s = 0.f;
    for (int t0 = 0; t0 < d.rows; t0 += 8) {
        float w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = ldg(d.a + (int64_t)min(t0 + k, d.rows - 1) * d.ld + j);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (t0 + k < d.rows) s += w[k];
    }
    const float lam = fmaf(beta, ldg(d.out + j), (1.0f - beta) * s);
    if (!__builtin_isfinite(lam)) stg(flag, 1u);
    stg(d.out + j, lam);
}

// P = diag(d_L) G diag(d_R) over row tiles of diag_scale_rows(n) rows
__global__ __launch_bounds__(256) void diag_scale_kernel(const DiagDesc* __restrict__ descs,
                                                         const int* __restrict__ prefix, int ndesc,
                                                         const IoEntry* __restrict__ io) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const DiagDesc& d = descs[item];
    const int rows = diag_scale_rows(d.n);
    const int r0 = (blockIdx.x - prefix[item]) * rows;
    const int r1 = min(r0 + rows, d.m);
    const float* __restrict__ G = io[d.blk].G;
    float* __restrict__ P = io[d.blk].P;
    const int64_t ldg_ = io[d.blk].ldg, ldp = io[d.blk].ldp;
    for (int i = r0; i < r1; ++i) {
        const float dl = ldg(d.d_l + i);
        for (int j = threadIdx.x; j < d.n; j += 256)
            stg(P + (int64_t)i * ldp + j, dl * ldg(G + (int64_t)i * ldg_ + j) * ldg(d.d_r + j));
    }
}

}  // namespace

hipError_t launch_diag_partials(const DiagDesc* descs, const int* prefix, int ndesc, int ntiles,
                                const IoEntry* io, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(diag_partials_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, io);
    return hipGetLastError();
}

hipError_t launch_diag_ema(const VecDesc* descs, const int* prefix, int ndesc, int ntiles, float beta,
                           uint32_t* flag, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(diag_ema_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, beta, flag);
    return hipGetLastError();
}

hipError_t launch_diag_scale(const DiagDesc* descs, const int* prefix, int ndesc, int ntiles,
                             const IoEntry* io, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(diag_scale_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, io);
    return hipGetLastError();
}

}  // namespace s4
