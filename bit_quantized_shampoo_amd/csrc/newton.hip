// Elementwise steps of the coupled Newton iteration for the inverse 4th root ("Shampoo --
// Second-Order Optimizer", section "Computing the inverse fourth root", the matrix-
// multiply route): scale the damped factor by its Frobenius norm, form the factor
// F = (5 I - M) / 4 each iteration, and scale the result back.  The products
// X F, F F, F2 F2 and F4 M run on the MFMA GEMM.
//
// All kernels work on row tiles of p x p matrices (one NewtonDesc per matrix); a
// workgroup covers fill_rows(p) whole rows and its lanes stride the columns.
#include "kernels.hpp"

namespace s4 {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ int tile_rows(int p) { return fill_rows(p); }

// partial sums of squares of (A + eps I) over a row tile -> parts[tile]
__global__ __launch_bounds__(256) void newton_norm_kernel(const NewtonDesc* __restrict__ descs,
                                                          const int* __restrict__ prefix, int ndesc,
                                                          float eps) {
    __shared__ float red[4];
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const NewtonDesc& d = descs[item];
    const int tile = blockIdx.x - prefix[item];
    const int p = d.p;
    const int r0 = tile * tile_rows(p), r1 = min(r0 + tile_rows(p), p);
    float s = 0.f;
    for (int i = r0; i < r1; ++i)
        for (int j = threadIdx.x; j < p; j += 256) {
            const float v = ldg(d.A + (int64_t)i * d.lda + j) + (i == j ? eps : 0.f);
            s = fmaf(v, v, s);
        }
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) stg(d.parts + tile, (red[0] + red[1]) + (red[2] + red[3]));
}

// c = sqrt(sum of the matrix's partials) into its scale slot (one workgroup per matrix,
// fixed order)
__global__ __launch_bounds__(64) void newton_scale_kernel(const NewtonDesc* __restrict__ descs, int ndesc) {
    const NewtonDesc& d = descs[blockIdx.x];
    const int ntiles = (d.p + tile_rows(d.p) - 1) / tile_rows(d.p);
    float s = 0.f;
    for (int t = threadIdx.x; t < ntiles; t += 64) s += ldg(d.parts + t);
    s = wave_sum(s);
    if (threadIdx.x == 0) stg(d.scale, sqrtf(s));
}

// mode 0: dst = (A + eps I) / c (from the caller's lda to contiguous) and ident = I
// mode 1: dst = 1.25 I - 0.25 src (the factor F = (5 I - M) / 4)
// mode 2: out (caller's ldo) = c^(-1/4) src
__global__ __launch_bounds__(256) void newton_elem_kernel(const NewtonDesc* __restrict__ descs,
                                                          const int* __restrict__ prefix, int ndesc,
                                                          int mode, float eps) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const NewtonDesc& d = descs[item];
    const int tile = blockIdx.x - prefix[item];
    const int p = d.p;
    const int r0 = tile * tile_rows(p), r1 = min(r0 + tile_rows(p), p);
    const float c = ldg(d.scale);
    const float rc = 1.f / c;
    const float root = 1.f / sqrtf(sqrtf(c));
    for (int i = r0; i < r1; ++i)
        for (int j = threadIdx.x; j < p; j += 256) {
            const float diag = (i == j) ? 1.f : 0.f;
            if (mode == 0) {
                const float v = ldg(d.A + (int64_t)i * d.lda + j) + diag * eps;
                stg(d.dst + (int64_t)i * p + j, v * rc);
                stg(d.ident + (int64_t)i * p + j, diag);
            } else if (mode == 1) {
                stg(d.dst + (int64_t)i * p + j, fmaf(-0.25f, ldg(d.src + (int64_t)i * p + j), 1.25f * diag));
            } else {
                stg(d.out + (int64_t)i * d.ldo + j, root * ldg(d.src + (int64_t)i * p + j));
            }
        }
}

}  // namespace

hipError_t launch_newton_norm(const NewtonDesc* descs, const int* prefix, int ndesc, int ntiles, float eps,
                              hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(newton_norm_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, eps);
    return hipGetLastError();
}

hipError_t launch_newton_scale(const NewtonDesc* descs, int ndesc, hipStream_t stream) {
    if (ndesc <= 0) return hipSuccess;
    S4_LAUNCH(newton_scale_kernel, dim3(ndesc), dim3(64), 0, stream, descs, ndesc);
    return hipGetLastError();
}

hipError_t launch_newton_elem(const NewtonDesc* descs, const int* prefix, int ndesc, int ntiles, int mode,
                              float eps, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(newton_elem_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, mode, eps);
    return hipGetLastError();
}

}  // namespace s4
