// Pieces shared by the two matrix-product kernels (fp32 operands on the fp32 matrix
// cores, gemm.hip; fp32 operands split into three bf16 planes on the bf16 matrix cores,
// gemm_x3.hip): the tile decode of a descriptor's workgroup index and the epilogue that
// writes a workgroup's 32 x 32 accumulator blocks.  Both kernels keep their accumulators
// in the layout of the 32 x 32 MFMA result: register r of lane (h = lane / 32, l32)
// holds row 8 (r / 4) + 4 h + (r % 4), column l32 of its block.
#pragma once

#include "kernels.hpp"

namespace s4 {

// Operand loads are branch-free: every address is clamped into the operand and
// out-of-range elements are zeroed with an AND on the loaded bits.  (A select on a
// loaded value is turned into a branch around the load with a wait for it inside,
// which serializes the loads of a tile.)
__device__ __forceinline__ float keep_if(float v, bool keep) {
    return __uint_as_float(__float_as_uint(v) & (keep ? 0xffffffffu : 0u));
}

// Workgroups of a launch that are resident at once (two per CU on the 256 CUs).
constexpr int GEMM_RESIDENT = 512;

// Logical tile index of this workgroup.  Workgroups go to the eight XCDs round robin
// (workgroup b to XCD b % 8), and each XCD has its own L2.  A launch that is resident at
// once gives XCD x the contiguous range [x n / 8, (x + 1) n / 8) of its tiles (the
// remainder, under eight, keeps its place), so the tiles one L2 serves share operand
// panels; a larger launch keeps the plain order (its first wave would otherwise stream
// eight distant regions of the batch at once).
__device__ __forceinline__ int gemm_block_index() {
    const int b = blockIdx.x, n = gridDim.x;
    if (n > GEMM_RESIDENT) return b;
    const int n8 = n >> 3;
    return b < 8 * n8 ? (b & 7) * n8 + (b >> 3) : b;
}

// Output tile of workgroup t of a descriptor: split-K chunk ks, tile (tile_m, tile_n).
// Symmetric products enumerate the tiles on and above the diagonal column by column:
// t = tn (tn + 1) / 2 + tm with tm <= tn.  Other products take the tiles column by column
// (tile_m fastest), or, in a launch resident at once, in groups of up to eight tile rows
// (rows fastest within a group), so a run of 64 consecutive tiles covers 8 x 8 of them.
template <int BM, int BN>
__device__ __forceinline__ void decode_tile(const GemmDesc& dsc, int t, int& ks, int& tile_m, int& tile_n) {
    const int tiles_m = dsc.tiles_m;
    const bool sym = (dsc.flags & GEMM_F_SYM) != 0;
    const int tiles_mn = sym ? tiles_m * (tiles_m + 1) / 2 : tiles_m * ((dsc.N + BN - 1) / BN);
    ks = t / tiles_mn;
    const int tmn = t - ks * tiles_mn;
    if (sym) {
        int tn = (int)((sqrtf(8.f * (float)tmn + 1.f) - 1.f) * 0.5f);
        while ((tn + 1) * (tn + 2) / 2 <= tmn) ++tn;
        while (tn * (tn + 1) / 2 > tmn) --tn;
        tile_n = tn;
        tile_m = tmn - tn * (tn + 1) / 2;
    } else if ((int)gridDim.x <= GEMM_RESIDENT) {
        const int tiles_n = (dsc.N + BN - 1) / BN;
        const int g = tmn / (8 * tiles_n);
        const int gh = min(8, tiles_m - 8 * g);
        const int local = tmn - 8 * g * tiles_n;
        tile_m = 8 * g + local % gh;
        tile_n = local / gh;
    } else {
        tile_m = tmn % tiles_m;
        tile_n = tmn / tiles_m;
    }
}

// Epilogue of a workgroup of WM x WN waves, each with TM x TN accumulator blocks:
// D = alpha * acc [* row scale][* column scale] + beta * C, the transposed block too for
// an off-diagonal tile of a symmetric product (mirror), or (GEMM_F_COLDOT) one partial
// row per tile: D[tile_m][col] = alpha * sum over the tile's rows of acc * C.
// lds_a / lds_b: LDS free for reuse (after the K loop's last barrier), at least
// max(WM * BN, 2 * 32 * 33) floats each.  Every thread of the workgroup calls it (the
// column-dot form has one workgroup barrier).
template <int WM, int WN, int TM, int TN>
__device__ __forceinline__ void gemm_epilogue(const floatx16 (&acc)[TM][TN], const GemmDesc& dsc, float* __restrict__ D,
                                              int64_t ldd, int tile_m, int row0, int col0, bool mirror,
                                              float* __restrict__ lds_a, float* __restrict__ lds_b, int tid) {
    constexpr int BN = WN * TN * 32;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int wave_m = wv % WM;
    const int wave_n = wv / WM;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int M = dsc.M, N = dsc.N;
    const float alpha = dsc.alpha, beta = dsc.beta;
    const float* __restrict__ C = dsc.C;
    const int64_t ldc = dsc.ldc;

    if (dsc.flags & GEMM_F_COLDOT) {
        float* red = lds_a;
#pragma unroll
        for (int n = 0; n < TN; ++n) {
            const int lcol = wave_n * TN * 32 + n * 32 + l32;
            const int col = col0 + lcol;
            float s = 0.f;
            const int colc = min(col, N - 1);
#pragma unroll
            for (int m = 0; m < TM; ++m) {
                float cv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row0 + wave_m * TM * 32 + m * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
                    cv[r] = ldg(C + (int64_t)min(row, M - 1) * ldc + colc);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row0 + wave_m * TM * 32 + m * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
                    s += acc[m][n][r] * keep_if(cv[r], row < M && col < N);
                }
                __builtin_amdgcn_sched_barrier(0);   // one 32 x 32 block's C values live at a time
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
                if (col < N) stg(D + (int64_t)tile_m * ldd + col, alpha * s);
            }
        }
        return;
    }

    const float* __restrict__ rs = dsc.rscale;
    const float* __restrict__ cs = dsc.cscale;
    // the C, row-scale and column-scale values of a 32 x 32 block are loaded (clamped
    // addresses) before any is used, absent ones from D in their place and replaced by
    // bit masks; stores are predicated on the bounds
    const float* __restrict__ cp = (beta != 0.f) ? C : D;
    const int64_t ldcp = (beta != 0.f) ? ldc : ldd;
    const float* __restrict__ rsp = rs ? rs : D;
    const uint32_t rsm = rs ? 0xffffffffu : 0u;
    const float* __restrict__ csp = cs ? cs : D;
    const uint32_t csm = cs ? 0xffffffffu : 0u;
#pragma unroll
    for (int n = 0; n < TN; ++n) {
        const int col = col0 + wave_n * TN * 32 + n * 32 + l32;
        const int colc = min(col, N - 1);
        const float csv = __uint_as_float((__float_as_uint(ldg(csp + colc)) & csm) | (0x3f800000u & ~csm));
#pragma unroll
        for (int m = 0; m < TM; ++m) {
            float cv[16], rv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + wave_m * TM * 32 + m * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
                const int rowc = min(row, M - 1);
                cv[r] = keep_if(ldg(cp + (int64_t)rowc * ldcp + colc), beta != 0.f);
                rv[r] = __uint_as_float((__float_as_uint(ldg(rsp + rowc)) & rsm) | (0x3f800000u & ~rsm));
            }
            float v[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + wave_m * TM * 32 + m * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
                v[r] = fmaf(beta, cv[r], alpha * acc[m][n][r] * rv[r] * csv);
                if (row < M && col < N) stg(D + (int64_t)row * ldd + col, v[r]);
            }
            if (mirror) {
                // the transposed block through a per-wave LDS tile, stored with one row
                // per half-wave (coalesced)
                float* tl = (wv < 2 ? lds_a : lds_b) + (wv & 1) * (32 * 33);
#pragma unroll
                for (int r = 0; r < 16; ++r) tl[((r >> 2) * 8 + h * 4 + (r & 3)) * 33 + l32] = v[r];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const int r0b = row0 + wave_m * TM * 32 + m * 32;
                const int c0b = col0 + wave_n * TN * 32 + n * 32;
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    const int g = 2 * s + h;                    // column of the block -> row of D
                    const float tv = tl[l32 * 33 + g];
                    if (c0b + g < M && r0b + l32 < N) stg(D + (int64_t)(c0b + g) * ldd + r0b + l32, tv);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
            // one 32 x 32 block at a time: keeps the next block's loads from being
            // hoisted here (their registers would cap the kernel's occupancy)
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

}  // namespace s4
