// Householder panel factorization for the warm-started eigen refresh
// (subspace iteration P = L~ V, P = Q R with diag(R) >= 0; the root is then
// formed from eigenvectors, "Shampoo -- Second-Order Optimizer", section
// "Rotation, not just rescaling").
//
// The QR of a p x p matrix is blocked by panels of nb = 32 columns.  This kernel
// factors one panel (rows c0..p-1, columns c0..c0+nb-1) per workgroup; the panels
// of every matrix of a batch with the same panel index run in one launch.  The
// trailing update and the explicit Q accumulation are matrix products done by the
// MFMA GEMM in compact WY form: the panel's reflectors H_0..H_{nb-1} multiply to
// I - V T V^T, and the kernel emits V (explicit unit-lower) and Y = V T.
//
// Work layout (512 threads = 8 waves): lane bits 0..4 pick the column, the 16
// half-waves each own every 16th row.  A dot product v^T A[:, c] is then a
// per-lane running sum over the lane's rows followed by a 16-way LDS reduction, no
// cross-lane shuffles.  Each reflector step is: scalars (one thread), reflector +
// all dot products (one pass over the panel), update of the later columns (one
// pass, which also accumulates the next column's sum of squares), 4 barriers.
// Panels up to PANEL_LDS_MAX_ROWS rows (bounded by the device's LDS) are staged
// in LDS with a pitch of 33 floats; taller panels are worked in place in global
// memory (L2-resident).
//
// Reflector (LAPACK-style): for x = column j below and on the diagonal,
// alpha = x_0, sigma^2 = |x_1..|^2; sigma^2 == 0 gives tau = 0 (H = I) and
// R_jj = alpha; otherwise beta = -sign(alpha) |x|, tau = (beta - alpha) / beta,
// v = [1, x_1.. / (alpha - beta)], R_jj = beta.  The norm is computed unscaled
// and recomputed with a power-of-two scaling when it would over- or underflow.
#include "kernels.hpp"

namespace s4 {

namespace {

constexpr int NSLOT = 16;

__device__ __forceinline__ int first_row(int j, int slot) {
    return j + ((slot - (j & (NSLOT - 1)) + NSLOT) & (NSLOT - 1));
}

template <bool IN_LDS>
__global__ __launch_bounds__(PANEL_THREADS) void panel_kernel(const PanelDesc* __restrict__ descs) {
    extern __shared__ float smem[];
    const PanelDesc d = descs[blockIdx.x];
    const int h = d.h, nb = d.nb;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c = lane & 31;
    const int slot = (tid >> 6) * 2 + (lane >> 5);
    const int64_t pitch = IN_LDS ? 33 : d.ld;
    float* __restrict__ S = IN_LDS ? smem : d.A + (int64_t)d.c0 * d.ld + d.c0;
    float* red = smem + (IN_LDS ? (size_t)h * 33 : 0);   // [NSLOT][32]
    float* Tm = red + NSLOT * 32;                        // [32][32]
    float* sv = Tm + 32 * 32;                            // [32]
    float* scal = sv + 32;                               // tau, beta, 1/(alpha-beta)

    if (IN_LDS) {
        for (int idx = tid; idx < h * 32; idx += PANEL_THREADS) {
            const int r = idx >> 5, cc = idx & 31;
            S[r * 33 + cc] = (cc < nb) ? d.A[(int64_t)(d.c0 + r) * d.ld + d.c0 + cc] : 0.f;
        }
    }
    for (int idx = tid; idx < 32 * 32; idx += PANEL_THREADS) Tm[idx] = 0.f;
    __syncthreads();

    {   // sum of squares of column 0 below the diagonal
        float ssq = 0.f;
        if (c == 0)
            for (int r = first_row(1, slot); r < h; r += NSLOT) {
                const float x = S[r * pitch];
                ssq += x * x;
            }
        red[slot * 32 + c] = ssq;
    }
    __syncthreads();

    for (int j = 0; j < nb; ++j) {
        if (tid == 0) {
            float sigma2 = 0.f;
            for (int q = 0; q < NSLOT; ++q) sigma2 += red[q * 32 + j];
            const float alpha = S[(int64_t)j * pitch + j];
            float nrm = sqrtf(alpha * alpha + sigma2);
            if (sigma2 != 0.f && (!__builtin_isfinite(nrm) || sigma2 < 1e-30f)) {
                // rescale by a power of two so the squares neither over- nor underflow
                float mx = fabsf(alpha);
                for (int r = j + 1; r < h; ++r) mx = fmaxf(mx, fabsf(S[(int64_t)r * pitch + j]));
                int e;
                frexpf(mx, &e);
                float ss = 0.f;
                for (int r = j; r < h; ++r) {
                    const float x = ldexpf(S[(int64_t)r * pitch + j], -e);
                    ss += x * x;
                }
                nrm = ldexpf(sqrtf(ss), e);
            }
            float tau, beta, sc;
            if (sigma2 == 0.f) {
                tau = 0.f; beta = alpha; sc = 0.f;
            } else {
                beta = (alpha >= 0.f) ? -nrm : nrm;
                tau = (beta - alpha) / beta;
                sc = 1.f / (alpha - beta);
            }
            scal[0] = tau; scal[1] = beta; scal[2] = sc;
            d.rdiag[d.c0 + j] = beta;
        }
        __syncthreads();
        const float tau = scal[0];
        const float sc = scal[2];

        // reflector v (column j) and the dots s_c = sum_{r >= j} v_r S[r][c]
        float part = 0.f;
        for (int r = first_row(j, slot); r < h; r += NSLOT) {
            const float sj = S[(int64_t)r * pitch + j];
            const float vr = (r == j) ? 1.f : sj * sc;
            const float x = (c < nb) ? S[(int64_t)r * pitch + c] : 0.f;
            part += vr * x;
            if (c == j && r > j) S[(int64_t)r * pitch + j] = vr;
        }
        red[slot * 32 + c] = part;
        __syncthreads();
        if (tid < 32) {
            float s = 0.f;
            for (int q = 0; q < NSLOT; ++q) s += red[q * 32 + tid];
            sv[tid] = s;
        }
        __syncthreads();

        // apply H_j to the later columns; accumulate the next column's sum of squares
        float ssq = 0.f;
        if (c > j && c < nb) {
            const float f = tau * sv[c];
            for (int r = first_row(j, slot); r < h; r += NSLOT) {
                const float vr = (r == j) ? 1.f : S[(int64_t)r * pitch + j];
                const float x = S[(int64_t)r * pitch + c] - f * vr;
                S[(int64_t)r * pitch + c] = x;
                if (r > j + 1) ssq += x * x;
            }
        }
        // column j of T: T[0:j, j] = -tau T[0:j, 0:j] s[0:j], T[j][j] = tau
        if (tid < j) {
            float acc = 0.f;
            for (int l = tid; l < j; ++l) acc += Tm[tid * 32 + l] * sv[l];
            Tm[tid * 32 + j] = -tau * acc;
        }
        if (tid == 32) Tm[j * 32 + j] = tau;
        red[slot * 32 + c] = ssq;
        __syncthreads();
    }

    // V (explicit unit-lower, zero beyond nb) and Y = V T, both [h, 32]
    for (int idx = tid; idx < h * 32; idx += PANEL_THREADS) {
        const int r = idx >> 5, cc = idx & 31;
        float y = 0.f, vrc = 0.f;
        if (cc < nb) {
            vrc = (r > cc) ? S[(int64_t)r * pitch + cc] : (r == cc ? 1.f : 0.f);
            const int imax = (cc < r) ? cc : r;   // V[r][i] = 0 for i > r
            for (int i = 0; i <= imax; ++i) {
                const float vri = (r > i) ? S[(int64_t)r * pitch + i] : 1.f;
                y += vri * Tm[i * 32 + cc];
            }
        }
        d.V[idx] = vrc;
        d.Y[idx] = y;
    }
}

}  // namespace

size_t panel_lds_bytes(bool in_lds, int max_h) {
    const size_t scratch = (size_t)(NSLOT * 32 + 32 * 32 + 32 + 4) * sizeof(float);
    return scratch + (in_lds ? (size_t)max_h * 33 * sizeof(float) : 0);
}

hipError_t launch_panel(bool in_lds, const PanelDesc* descs, int ndesc, int max_h,
                        hipStream_t stream) {
    if (ndesc <= 0) return hipSuccess;
    const size_t lds = panel_lds_bytes(in_lds, max_h);
    if (in_lds) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&panel_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        hipLaunchKernelGGL(panel_kernel<true>, dim3(ndesc), dim3(PANEL_THREADS), lds, stream, descs);
    } else {
        hipLaunchKernelGGL(panel_kernel<false>, dim3(ndesc), dim3(PANEL_THREADS), lds, stream, descs);
    }
    return hipGetLastError();
}

}  // namespace s4
