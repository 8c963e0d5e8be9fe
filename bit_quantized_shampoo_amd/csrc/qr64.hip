// Float64 pieces of the statistics update (the float64 refresh): Householder panels of
// the warm-started QR, the Rayleigh quotients and the float32 <-> float64 conversions.
//  * panel64:   one workgroup per h x nb panel (nb <= 32) of a p x p matrix, in place in
//               global memory: for each column j the reflector H_j = I - tau v v^T with
//               v_j = 1 that zeroes the column below the diagonal (the elementary
//               reflector of LAPACK's dlarfg: beta = -sign(alpha) |x|, tau = (beta -
//               alpha) / beta, H = I when the column is already zero below the diagonal),
//               applied to the panel's remaining columns; then T of the compact WY form
//               (H_0 ... H_{nb-1} = I - V T V^T, forward column by column as LAPACK's
//               dlarft) and Y = V T.  The column dots of a step, its sum of squares
//               included, are one fixed-order workgroup reduction.
//  * coldot64:  lam_j = max(sum_i Q[i][j] W[i][j], 0) (float32 out), W = L~ Q;
//  * ident64:   Q = diag(sign(R_jj)) (0 -> +), the start of the backward accumulation;
//  * cvt:       float32 -> float64 and back.
#include "kernels.hpp"

namespace s4 {

namespace {

constexpr int P64_THREADS = 256;

// Fixed-order sum of one value per thread over the workgroup: lane butterflies, then the
// four wave sums in order.  `red` holds 4 doubles per value slot.
__device__ __forceinline__ double wave_sum64(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__global__ __launch_bounds__(P64_THREADS) void panel64_kernel(const Panel64Desc* __restrict__ descs) {
    const Panel64Desc& d = descs[blockIdx.x];
    __shared__ double red[4][33];
    __shared__ double wcol[33];
    __shared__ double tau_s[32];
    __shared__ double T[32][33];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int h = d.h, nb = d.nb;
    double* __restrict__ A = d.A + (int64_t)d.c0 * d.ld + d.c0;   // panel's top-left element
    const int64_t ld = d.ld;
    double* __restrict__ V = d.V;
    const int64_t vld = d.vld;
    for (int j = 0; j < nb; ++j) {
        // partial dots of column j (rows j+1..) with columns j..nb-1 of the panel
        double part[32];
#pragma unroll
        for (int c = 0; c < 32; ++c) part[c] = 0.0;
        for (int r = j + 1 + tid; r < h; r += P64_THREADS) {
            const double* row = A + (int64_t)r * ld;
            const double x = row[j];
#pragma unroll
            for (int c = 0; c < 32; ++c)
                if (c >= j && c < nb) part[c] = fma(x, row[c], part[c]);
        }
#pragma unroll
        for (int c = 0; c < 32; ++c)
            if (c >= j && c < nb) {   // uniform: every lane of the wave takes it
                const double s = wave_sum64(part[c]);
                if (lane == 0) red[wv][c] = s;
            }
        __syncthreads();
        if (tid < nb && tid >= j) wcol[tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
        __syncthreads();
        // reflector of column j: sigma = |x below the diagonal|^2, alpha = A[j][j]
        const double sigma = wcol[j];
        const double alpha = A[(int64_t)j * ld + j];
        double tau = 0.0, beta = alpha, scale = 0.0;
        if (sigma > 0.0) {
            const double nrm = sqrt(fma(alpha, alpha, sigma));
            beta = alpha >= 0.0 ? -nrm : nrm;
            tau = (beta - alpha) / beta;
            scale = 1.0 / (alpha - beta);
        }
        // w_c = v^T A[:, c] = A[j][c] + scale * dot_c for the remaining columns
        double w[32];
#pragma unroll
        for (int c = 0; c < 32; ++c)
            w[c] = (c > j && c < nb) ? tau * fma(scale, wcol[c], A[(int64_t)j * ld + min(c, nb - 1)]) : 0.0;
        __syncthreads();   // every thread has read wcol and row j before they change
        for (int r = j + tid; r < h; r += P64_THREADS) {
            double* row = A + (int64_t)r * ld;
            const double v = (r == j) ? 1.0 : scale * row[j];
#pragma unroll
            for (int c = 0; c < 32; ++c)
                if (c > j && c < nb) row[c] = fma(-w[c], v, row[c]);
            V[(int64_t)r * vld + j] = v;
            if (r == j) row[j] = beta;
        }
        // V above the diagonal of column j is zero
        for (int r = tid; r < j; r += P64_THREADS) V[(int64_t)r * vld + j] = 0.0;
        if (tid == 0) {
            tau_s[j] = tau;
            d.rdiag[d.c0 + j] = beta;
        }
        __syncthreads();
    }
    // columns nb..31 of V and Y are zero (a short last panel)
    for (int idx = tid; idx < h * (32 - nb); idx += P64_THREADS) {
        const int r = idx / (32 - nb), c = nb + idx % (32 - nb);
        V[(int64_t)r * vld + c] = 0.0;
        d.Y[(int64_t)r * vld + c] = 0.0;
    }
    __syncthreads();
    // T (upper triangular): T[j][j] = tau_j, T[0:j, j] = -tau_j T[0:j, 0:j] (V[:, 0:j]^T v_j)
    // Gram entries g[a][b] = v_a^T v_b over the panel's rows, a < b
    __shared__ double G[32][33];
    for (int a = 0; a < nb; ++a) {
        double part[32];
#pragma unroll
        for (int b = 0; b < 32; ++b) part[b] = 0.0;
        for (int r = tid; r < h; r += P64_THREADS) {
            const double* vr = V + (int64_t)r * vld;
            const double va = vr[a];
#pragma unroll
            for (int b = 0; b < 32; ++b)
                if (b > a && b < nb) part[b] = fma(va, vr[b], part[b]);
        }
#pragma unroll
        for (int b = 0; b < 32; ++b)
            if (b > a && b < nb) {
                const double s = wave_sum64(part[b]);
                if (lane == 0) red[wv][b] = s;
            }
        __syncthreads();
        if (tid > a && tid < nb) G[a][tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
        __syncthreads();
    }
    if (tid == 0) {
        for (int j = 0; j < nb; ++j) {
            T[j][j] = tau_s[j];
            for (int i = 0; i < j; ++i) {
                double s = 0.0;
                for (int l = i; l < j; ++l) s = fma(T[i][l], G[l][j], s);
                T[i][j] = -tau_s[j] * s;
            }
            for (int i = j + 1; i < 32; ++i) T[i][j] = 0.0;
        }
    }
    __syncthreads();
    // Y = V T (rows of V times the upper triangle)
    for (int r = tid; r < h; r += P64_THREADS) {
        const double* vr = V + (int64_t)r * vld;
        double vrow[32];
#pragma unroll
        for (int a = 0; a < 32; ++a) vrow[a] = a < nb ? vr[a] : 0.0;
        for (int b = 0; b < nb; ++b) {
            double s = 0.0;
#pragma unroll
            for (int a = 0; a < 32; ++a)
                if (a <= b) s = fma(vrow[a], T[a][b], s);
            d.Y[(int64_t)r * vld + b] = s;
        }
    }
}

// lam_j = max(sum_i Q[i][j] W[i][j], 0), rows in order; one thread per column
__global__ __launch_bounds__(256) void coldot64_kernel(const Vec64Desc* __restrict__ descs,
                                                       const int* __restrict__ prefix, int ndesc,
                                                       uint32_t* __restrict__ flag) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const Vec64Desc& d = descs[item];
    const int j = (blockIdx.x - prefix[item]) * 256 + threadIdx.x;
    if (j >= d.p) return;
    double s = 0.0;
    for (int i = 0; i < d.p; ++i) s = fma(ldg(d.a + (int64_t)i * d.p + j), ldg(d.b + (int64_t)i * d.p + j), s);
    const float lam = (float)(s > 0.0 ? s : 0.0);
    if (!__builtin_isfinite(lam)) stg(flag, 1u);
    stg(d.f32 + j, lam);
}

// out = diag(sign(aux)) (0 -> +), p x p, rows of one workgroup
__global__ __launch_bounds__(256) void ident64_kernel(const Vec64Desc* __restrict__ descs,
                                                      const int* __restrict__ prefix, int ndesc) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const Vec64Desc& d = descs[item];
    const int i = blockIdx.x - prefix[item];
    const double one = ldg(d.a + i) < 0.0 ? -1.0 : 1.0;
    for (int j = threadIdx.x; j < d.p; j += 256) stg(d.out + (int64_t)i * d.p + j, (i == j) ? one : 0.0);
}

// float32 <-> float64 over n = p * p elements (dir 0: f32 -> f64, 1: f64 -> f32)
__global__ __launch_bounds__(256) void cvt_kernel(const Vec64Desc* __restrict__ descs,
                                                  const int* __restrict__ prefix, int ndesc, int dir) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const Vec64Desc& d = descs[item];
    const int64_t n = (int64_t)d.p * d.p;
    const int64_t base = (int64_t)(blockIdx.x - prefix[item]) * CVT_TILE;
    for (int64_t e = base + threadIdx.x; e < base + CVT_TILE && e < n; e += 256) {
        if (dir == 0) stg(d.out + e, (double)ldg(d.f32 + e));
        else stg(d.f32 + e, (float)ldg(d.a + e));
    }
}

}  // namespace

hipError_t launch_panel64(const Panel64Desc* descs, int ndesc, hipStream_t stream) {
    if (ndesc <= 0) return hipSuccess;
    S4_LAUNCH(panel64_kernel, dim3(ndesc), dim3(P64_THREADS), 0, stream, descs);
    return hipGetLastError();
}

hipError_t launch_coldot64(const Vec64Desc* descs, const int* prefix, int ndesc, int ntiles, uint32_t* flag,
                           hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(coldot64_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, flag);
    return hipGetLastError();
}

hipError_t launch_ident64(const Vec64Desc* descs, const int* prefix, int ndesc, int ntiles, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(ident64_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc);
    return hipGetLastError();
}

hipError_t launch_cvt(const Vec64Desc* descs, const int* prefix, int ndesc, int ntiles, int dir,
                      hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(cvt_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, dir);
    return hipGetLastError();
}

}  // namespace s4
