// Small bandwidth-bound kernels of the step.
//  * root scaling:  d_i = (lam_i + eps)^(-1/4) ("Shampoo -- Second-Order Optimizer",
//                   "Computing the inverse fourth root": damping before rooting);
//  * rayleigh reduce: lam_j = max(sum_r Q[r][j] (L~ Q)[r][j], 0) from the per-tile
//                   partial sums the column-dot GEMM epilogue leaves (fixed order);
//  * identity fill / sign flip: Q starts as I for the forward accumulation of
//                   the reflectors and its column j is finally multiplied by
//                   sign(R_jj) (0 -> +), so that diag(R) >= 0; the backward
//                   accumulation (Q <- H_b Q, last block first) starts instead from
//                   diag(sign(R_jj)), which gives the flipped Q with no second pass;
//  * identity state: U = I coded exactly (code 15 on the diagonal, 7 elsewhere,
//                   scale 1 for blocks holding a diagonal element, else 0), lam = 0,
//                   root = (I, d = 1).
#include "kernels.hpp"

namespace s4 {

namespace {

__global__ __launch_bounds__(256) void root_scaling_kernel(const VecDesc* __restrict__ descs,
                                                           const int* __restrict__ prefix, int ndesc,
                                                           float eps, uint32_t* __restrict__ flag) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const VecDesc& d = descs[item];
    const int i = (blockIdx.x - prefix[item]) * 256 + threadIdx.x;
    if (i >= d.p) return;
    const float x = d.a[i] + eps;
    if (!__builtin_isfinite(x)) flag[0] = 1u;
    d.out[i] = 1.0f / sqrtf(sqrtf(x));
}

__global__ __launch_bounds__(256) void rayleigh_reduce_kernel(const VecDesc* __restrict__ descs,
                                                              const int* __restrict__ prefix, int ndesc,
                                                              uint32_t* __restrict__ flag) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const VecDesc& d = descs[item];
    const int j = (blockIdx.x - prefix[item]) * 256 + threadIdx.x;
    if (j >= d.p) return;
    // partial rows 16 at a time, all loads (clamped rows) issued before the sum, which
    // adds them in row order
    float t = 0.f;
    for (int r0 = 0; r0 < d.rows; r0 += 16) {
        float v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = ldg(d.a + (int64_t)min(r0 + k, d.rows - 1) * d.ld + j);
#pragma unroll
        for (int k = 0; k < 16; ++k)
            if (r0 + k < d.rows) t += v[k];
    }
    if (!__builtin_isfinite(t)) flag[0] = 1u;
    d.out[j] = t > 0.f ? t : 0.f;
}

// out = I, or with SIGNED diag(sign(aux)) (0 -> +) (p x p, leading dimension ld); a
// workgroup covers fill_rows(p) whole rows
template <bool SIGNED>
__global__ __launch_bounds__(256) void identity_fill_kernel(const VecDesc* __restrict__ descs,
                                                            const int* __restrict__ prefix, int ndesc) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const VecDesc& d = descs[item];
    const int p = d.p;
    const int rows = fill_rows(p);
    const int r0 = (blockIdx.x - prefix[item]) * rows;
    const int r1 = min(r0 + rows, p);
    for (int i = r0; i < r1; ++i) {
        float* __restrict__ row = d.out + (int64_t)i * d.ld;
        const float one = (SIGNED && d.aux[i] < 0.f) ? -1.f : 1.f;
        for (int j = threadIdx.x; j < p; j += 256) row[j] = (i == j) ? one : 0.f;
    }
}

// column j of out times sign(aux[j]) (0 counts as +), same row tiling.  A thread's
// elements of a chunk (FILL_TILE / 256 of them, strided by 256) are all loaded, at clamped
// addresses, before any is stored: a load-negate-store chain per element waited one
// memory round trip each.
__global__ __launch_bounds__(256) void sign_flip_kernel(const VecDesc* __restrict__ descs,
                                                        const int* __restrict__ prefix, int ndesc) {
    constexpr int PER = FILL_TILE / 256;
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const VecDesc& d = descs[item];
    const int p = d.p;
    const int rows = fill_rows(p);
    const int r0 = (blockIdx.x - prefix[item]) * rows;
    const int n = (min(r0 + rows, p) - r0) * p;       // elements of this row tile
    const int qs = 256 / p, rs = 256 % p;             // a stride of 256 elements in (row, col)
    for (int base = 0; base < n; base += PER * 256) {
        int i = (base + (int)threadIdx.x) / p, jj = (base + (int)threadIdx.x) % p;
        float v[PER], sg[PER];
        int64_t off[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const bool in = base + k * 256 + (int)threadIdx.x < n;
            const int ic = in ? r0 + i : r0, jc = in ? jj : 0;
            off[k] = (int64_t)ic * d.ld + jc;
            v[k] = ldg(d.out + off[k]);
            // out of range: +0 (no store), by a mask rather than a select on the load
            sg[k] = __uint_as_float(__float_as_uint(ldg(d.aux + jc)) & (in ? 0xffffffffu : 0u));
            i += qs;
            jj += rs;
            if (jj >= p) { jj -= p; ++i; }
        }
#pragma unroll
        for (int k = 0; k < PER; ++k)
            if (sg[k] < 0.f) stg(d.out + off[k], -v[k]);
    }
}

__global__ __launch_bounds__(256) void identity_state_kernel(const InitDesc* __restrict__ descs,
                                                             const int* __restrict__ prefix, int ndesc) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const InitDesc& d = descs[item];
    const int64_t p = d.p;
    const int64_t n = p * p;
    const int64_t nqb = (n + 63) / 64;
    const int64_t i = (int64_t)(blockIdx.x - prefix[item]) * 256 + threadIdx.x;
    if (d.kind == INIT_DIAG) {
        // diagonal side: no eigenvectors
    } else if (i < nqb && d.kind == INIT_FP32) {   // float32 U = I: 64 elements per thread
        float* u = reinterpret_cast<float*>(d.codes);
        float* ru = reinterpret_cast<float*>(d.rcodes);
        for (int e = 0; e < 64; ++e) {
            const int64_t idx = i * 64 + e;
            if (idx < n) {
                const float v = (idx % (p + 1)) == 0 ? 1.f : 0.f;
                u[idx] = v;
                ru[idx] = v;
            }
        }
    } else if (i < nqb) {
        bool any = false;
        uint32_t words[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t idx = i * 64 + w * 8 + e;
                const bool diag = idx < n && (idx % (p + 1)) == 0;
                any = any || diag;
                word |= (diag ? 15u : 7u) << (4 * e);
            }
            words[w] = word;
        }
        uint32_t* c = reinterpret_cast<uint32_t*>(d.codes) + i * 8;
        uint32_t* rc = reinterpret_cast<uint32_t*>(d.rcodes) + i * 8;
#pragma unroll
        for (int w = 0; w < 8; ++w) { c[w] = words[w]; rc[w] = words[w]; }
        d.scales[i] = any ? 1.f : 0.f;
        d.rscales[i] = any ? 1.f : 0.f;
    }
    if (i < p) {
        d.lam[i] = 0.f;
        d.d[i] = 1.f;
    }
}

// out = a for n = ld floats (16-byte vectors, scalar tail); with a flag, non-finite
// values raise it (the 32-bit state's stand-in for the quantizer's check)
__global__ __launch_bounds__(256) void copyf_kernel(const VecDesc* __restrict__ descs,
                                                    const int* __restrict__ prefix, int ndesc,
                                                    uint32_t* __restrict__ flag) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const VecDesc& d = descs[item];
    const int64_t n = d.ld;
    const int64_t base = (int64_t)(blockIdx.x - prefix[item]) * COPYF_TILE;
    const bool vec = ((reinterpret_cast<uintptr_t>(d.a) | reinterpret_cast<uintptr_t>(d.out)) & 15) == 0;
    bool finite = true;
    if (vec) {
        for (int64_t e = base + 4 * threadIdx.x; e < base + COPYF_TILE && e < n; e += 4 * 256) {
            if (e + 4 <= n) {
                const floatx4 v = ldg(reinterpret_cast<const floatx4*>(d.a + e));
                stg(reinterpret_cast<floatx4*>(d.out + e), v);
                finite = finite && __builtin_isfinite(v[0]) && __builtin_isfinite(v[1]) &&
                         __builtin_isfinite(v[2]) && __builtin_isfinite(v[3]);
            } else {
                for (int64_t k = e; k < n; ++k) {
                    const float v = ldg(d.a + k);
                    stg(d.out + k, v);
                    finite = finite && __builtin_isfinite(v);
                }
            }
        }
    } else {
        for (int64_t e = base + threadIdx.x; e < base + COPYF_TILE && e < n; e += 256) {
            const float v = ldg(d.a + e);
            stg(d.out + e, v);
            finite = finite && __builtin_isfinite(v);
        }
    }
    if (!finite && flag) stg(flag, 1u);
}

}  // namespace

hipError_t launch_copyf(const VecDesc* descs, const int* prefix, int ndesc, int ntiles, uint32_t* flag,
                        hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(copyf_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, flag);
    return hipGetLastError();
}

hipError_t launch_root_scaling(const VecDesc* descs, const int* prefix, int ndesc, int ntiles,
                               float eps, uint32_t* flag, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(root_scaling_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc,
                       eps, flag);
    return hipGetLastError();
}

hipError_t launch_rayleigh_reduce(const VecDesc* descs, const int* prefix, int ndesc, int ntiles,
                                  uint32_t* flag, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(rayleigh_reduce_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, flag);
    return hipGetLastError();
}

hipError_t launch_identity_fill(const VecDesc* descs, const int* prefix, int ndesc, int ntiles, bool with_signs,
                                hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    if (with_signs)
        S4_LAUNCH(identity_fill_kernel<true>, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc);
    else
        S4_LAUNCH(identity_fill_kernel<false>, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc);
    return hipGetLastError();
}

hipError_t launch_sign_flip(const VecDesc* descs, const int* prefix, int ndesc, int ntiles,
                            hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(sign_flip_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc);
    return hipGetLastError();
}

hipError_t launch_identity_state(const InitDesc* descs, const int* prefix, int ndesc, int ntiles,
                                 hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(identity_state_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc);
    return hipGetLastError();
}

}  // namespace s4
