// Grafting and the weight update after the preconditioner ("Shampoo -- Second-Order
// Optimizer", section "Grafting: borrow a step size that already works"): the step keeps
// Shampoo's direction P and takes its Frobenius norm, per block, from the step of a
// grafted method (SGD: G; Adam: bias-corrected m / (sqrt(v) + eps), moments updated here):
//     W <- W - lr * ||d_graft||_F / (||P||_F + eps_graft) * P.
//
// Both kernels are HBM streams over row tiles of every block (a workgroup covers
// graft_rows(n) whole rows, lanes stride the columns: coalesced rows of G, P, W, M, V).
//  * graft_norms: per tile, sum of d_graft^2 and of P^2 (wave butterflies, then the four
//    waves in order), written as two partials; Adam moments updated in the same pass.
//  * graft_apply: wave 0 sums the block's partials in a fixed order (tile-strided lanes,
//    then a butterfly), every workgroup derives the same scale and updates its rows of W.
// Bytes per element: SGD 8 + 12, Adam 24 + 12 (norm pass + update pass).
#include "kernels.hpp"

namespace s4 {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__global__ __launch_bounds__(256) void graft_norms_kernel(const GraftDesc* __restrict__ descs,
                                                          const int* __restrict__ prefix, int ndesc,
                                                          const IoEntry* __restrict__ io,
                                                          const GraftIo* __restrict__ gio, GraftParams prm,
                                                          uint32_t* __restrict__ flag) {
    __shared__ float red[8];
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const GraftDesc d = descs[item];
    const int tile = blockIdx.x - prefix[item];
    const int r0 = tile * d.rows;
    const int r1 = min(r0 + d.rows, d.m);
    const IoEntry e = io[d.blk];
    const GraftIo g = gio[d.blk];
    float sg = 0.f, sp = 0.f;
    for (int i = r0; i < r1; ++i) {
        const float* __restrict__ grow = e.G + (int64_t)i * e.ldg;
        const float* __restrict__ prow = e.P + (int64_t)i * e.ldp;
        for (int j = threadIdx.x; j < d.n; j += 256) {
            const float gv = ldg(grow + j);
            const float pv = ldg(prow + j);
            float dg = gv;
            if (prm.mode == 1) {
                const int64_t k = (int64_t)i * d.n + j;
                const float mv = fmaf(prm.beta1, ldg(g.M + k), (1.f - prm.beta1) * gv);
                const float vv = fmaf(prm.beta2, ldg(g.V + k), (1.f - prm.beta2) * (gv * gv));
                stg(g.M + k, mv);
                stg(g.V + k, vv);
                dg = (mv / prm.c1) / (sqrtf(vv / prm.c2) + prm.eps_adam);
            }
            sg = fmaf(dg, dg, sg);
            sp = fmaf(pv, pv, sp);
        }
    }
    sg = wave_sum(sg);
    sp = wave_sum(sp);
    const int wv = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[2 * wv] = sg;
        red[2 * wv + 1] = sp;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const float a = (red[0] + red[2]) + (red[4] + red[6]);
        const float b = (red[1] + red[3]) + (red[5] + red[7]);
        stg(d.parts + 2 * tile, a);
        stg(d.parts + 2 * tile + 1, b);
        if (!__builtin_isfinite(a) || !__builtin_isfinite(b)) stg(flag, 1u);
    }
}

__global__ __launch_bounds__(256) void graft_apply_kernel(const GraftDesc* __restrict__ descs,
                                                          const int* __restrict__ prefix, int ndesc,
                                                          const IoEntry* __restrict__ io,
                                                          const GraftIo* __restrict__ gio, GraftParams prm) {
    __shared__ float tot[2];
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const GraftDesc d = descs[item];
    const int tile = blockIdx.x - prefix[item];
    if (threadIdx.x < 64) {
        float a = 0.f, b = 0.f;
        for (int t = threadIdx.x; t < d.ntiles; t += 64) {
            a += ldg(d.parts + 2 * t);
            b += ldg(d.parts + 2 * t + 1);
        }
        a = wave_sum(a);
        b = wave_sum(b);
        if (threadIdx.x == 0) {
            tot[0] = a;
            tot[1] = b;
        }
    }
    __syncthreads();
    const float scale = prm.lr * (sqrtf(tot[0]) / (sqrtf(tot[1]) + prm.eps_graft));
    const int r0 = tile * d.rows;
    const int r1 = min(r0 + d.rows, d.m);
    const IoEntry e = io[d.blk];
    const GraftIo g = gio[d.blk];
    for (int i = r0; i < r1; ++i) {
        const float* __restrict__ prow = e.P + (int64_t)i * e.ldp;
        float* __restrict__ wrow = g.W + (int64_t)i * g.ldw;
        for (int j = threadIdx.x; j < d.n; j += 256) stg(wrow + j, fmaf(-scale, ldg(prow + j), ldg(wrow + j)));
    }
}

}  // namespace

hipError_t launch_graft_norms(const GraftDesc* descs, const int* prefix, int ndesc, int ntiles,
                              const IoEntry* io, const GraftIo* gio, GraftParams prm, uint32_t* flag,
                              hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(graft_norms_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, io, gio, prm, flag);
    return hipGetLastError();
}

hipError_t launch_graft_apply(const GraftDesc* descs, const int* prefix, int ndesc, int ntiles,
                              const IoEntry* io, const GraftIo* gio, GraftParams prm, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(graft_apply_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, io, gio, prm);
    return hipGetLastError();
}

}  // namespace s4
