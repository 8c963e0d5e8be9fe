// Householder panel factorization for the warm-started eigen refresh
// (subspace iteration P = L~ V, P = Q R with diag(R) >= 0; the root is then
// formed from eigenvectors, "Shampoo -- Second-Order Optimizer", section
// "Rotation, not just rescaling").
//
// The QR of a p x p matrix is blocked by panels of 32 columns.  This kernel
// factors one panel (rows c0..p-1, columns c0..c0+nb-1) per workgroup; the panels
// of every matrix of a batch with the same panel index run in one launch.  The
// trailing update and the accumulation of Q are matrix products done by the MFMA
// GEMM in compact WY form: the panel's reflectors H_0..H_{nb-1} multiply to
// I - V T V^T, and the kernel emits V (explicit unit-lower) and Y = V T.
//
// Work layout (512 threads = 8 waves): lane bits 0..4 pick the column, the 16
// half-waves each own every 16th row.  For panels up to 16*NR rows the panel
// lives in registers (NR values per lane); taller panels are worked in place in
// global memory (L2) with the same schedule.
//
// One reflector step needs a single barrier.  With x = column j and
// d_c = sum_{r >= j} x_r A[r][c] for every column c, the reflector is
// beta = -sign(alpha) sqrt(alpha^2 + sigma^2) (sigma^2 = |x below j|^2),
// tau = (beta - alpha) / beta, v = [1, x_{j+1..} / (alpha - beta)], and
// s_c = v^T A[:, c] = (d_c - beta A[j][c]) / (alpha - beta); sigma^2 = 0 gives
// H = I.  So one pass applies H_j to the later columns and, in the same sweep,
// accumulates the next column's d_c and sigma^2; the 16 half-wave partials meet
// in LDS (double-buffered by step parity) and every thread derives the next
// reflector's scalars itself.  The s_c (c < j) of every step are kept, and at the
// end one wave builds T row by row (T[c][j] = -tau_j sum_{c <= l < j} T[c][l] s_l,
// T[j][j] = tau_j) and the workgroup forms Y = V T with v_mfma_f32_32x32x2_f32.
//
// The panel is first scaled by a power of two so that its largest entry is in
// [0.5, 1): squares can neither overflow nor (for entries that matter) underflow,
// and V, tau and the signs of R are unchanged by the exact scaling.
#include "kernels.hpp"

namespace s4 {

namespace {

constexpr int NSLOT = 16;
constexpr int PW = 32;                 // panel width
constexpr int PART = NSLOT * 33;       // one partials buffer: [16][33]

// LDS layout (floats)
constexpr int OFF_PART = 0;                      // [2][16][33]
constexpr int OFF_ROWJ = OFF_PART + 2 * PART;    // [2][32]
constexpr int OFF_SALL = OFF_ROWJ + 64;          // [32][32] s vector of step j
constexpr int OFF_TAU = OFF_SALL + PW * PW;      // [32]
constexpr int OFF_T = OFF_TAU + PW;              // [32][33]
constexpr int OFF_RED = OFF_T + PW * 33;         // [16]
constexpr int OFF_VS = OFF_RED + 16;             // [hpad][33] staging of V (register variant)

struct Refl {
    float tau, beta, sc;
};

__device__ __forceinline__ Refl reflector(float alpha, float sigma2) {
    Refl s;
    if (sigma2 == 0.f) {
        s.tau = 0.f; s.beta = alpha; s.sc = 0.f;
    } else {
        const float nrm = sqrtf(alpha * alpha + sigma2);
        s.beta = (alpha >= 0.f) ? -nrm : nrm;
        s.tau = (s.beta - alpha) / s.beta;
        s.sc = 1.f / (alpha - s.beta);
    }
    return s;
}

// Reduce the partials of step `buf` for column c: d_c, sigma^2, alpha, A[j][c].
__device__ __forceinline__ void read_step(const float* smem, int buf, int j, int c, float& dc,
                                          float& sigma2, float& alpha, float& ajc) {
    const float* pb = smem + OFF_PART + buf * PART;
    dc = 0.f;
    sigma2 = 0.f;
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) {
        dc += pb[s * 33 + c];
        sigma2 += pb[s * 33 + 32];
    }
    alpha = smem[OFF_ROWJ + buf * 32 + j];
    ajc = smem[OFF_ROWJ + buf * 32 + c];
}

__device__ __forceinline__ float panel_max(float mx, float* smem, int lane, int wv) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) smem[OFF_RED + wv] = mx;
    __syncthreads();
    float m = 0.f;
#pragma unroll
    for (int w = 0; w < PANEL_THREADS / 64; ++w) m = fmaxf(m, smem[OFF_RED + w]);
    return m;
}

// T (upper triangular, nb x nb) from the kept s vectors and taus: one lane per row.
__device__ __forceinline__ void build_T(float* smem, int nb, int tid) {
    if (tid < PW) {
        const int c = tid;
        float trow[PW];
#pragma unroll
        for (int l = 0; l < PW; ++l) trow[l] = 0.f;
#pragma unroll
        for (int j = 0; j < PW; ++j) {
            if (j < nb) {
                const float tj = smem[OFF_TAU + j];
                if (c < j) {
                    float acc = 0.f;
#pragma unroll
                    for (int l = 0; l < PW; ++l)
                        if (l >= c && l < j) acc += trow[l] * smem[OFF_SALL + j * PW + l];
                    trow[j] = -tj * acc;
                } else if (c == j) {
                    trow[j] = tj;
                }
            }
        }
#pragma unroll
        for (int l = 0; l < PW; ++l) smem[OFF_T + c * 33 + l] = trow[l];
    }
}

// Y = V T for rows [0, h): V rows come from `vsrc` (pitch vpitch floats), T from LDS.
__device__ __forceinline__ void form_Y(const float* vsrc, int64_t vpitch, const float* smem, float* Y,
                                       int h, int tid) {
    const int lane = tid & 63, wv = tid >> 6, l32 = lane & 31, hh = lane >> 5;
    const int nchunk = (h + 31) / 32;
    for (int q = wv; q < nchunk; q += PANEL_THREADS / 64) {
        floatx16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        const int row = q * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < PW / 2; ++ks) {
            const int k = 2 * ks + hh;
            const float a = (row < h) ? vsrc[(int64_t)row * vpitch + k] : 0.f;
            const float b = smem[OFF_T + k * 33 + l32];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int orow = q * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
            if (orow < h) Y[(int64_t)orow * PW + l32] = acc[r];
        }
    }
}

template <int NR>
__global__ __launch_bounds__(PANEL_THREADS) void panel_reg_kernel(const PanelDesc* __restrict__ descs) {
    extern __shared__ float smem[];
    const PanelDesc d = descs[blockIdx.x];
    const int h = d.h, nb = d.nb;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c = lane & 31;
    const int wv = tid >> 6;
    const int slot = wv * 2 + (lane >> 5);
    const float* __restrict__ Ap = d.A + (int64_t)d.c0 * d.ld + d.c0;

    float x[NR], xc[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int r = slot + NSLOT * i;
        x[i] = (r < h && c < nb) ? Ap[(int64_t)r * d.ld + c] : 0.f;
    }
    {
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < NR; ++i) mx = fmaxf(mx, fabsf(x[i]));
        mx = panel_max(mx, smem, lane, wv);
        if (mx > 0.f) {
            int e;
            frexpf(mx, &e);
#pragma unroll
            for (int i = 0; i < NR; ++i) x[i] = ldexpf(x[i], -e);
        }
    }
    {   // dots and sigma^2 for column 0
        float pacc = 0.f, sg = 0.f, rj = 0.f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int r = slot + NSLOT * i;
            xc[i] = __shfl(x[i], 0, 32);
            if (r < h) {
                pacc += xc[i] * x[i];
                if (r > 0) sg += xc[i] * xc[i];
            }
            if (r == 0) rj = x[i];
        }
        smem[OFF_PART + slot * 33 + c] = pacc;
        if (c == 0) smem[OFF_PART + slot * 33 + 32] = sg;
        if (slot == 0) smem[OFF_ROWJ + c] = rj;
    }
    __syncthreads();

    for (int j = 0; j < nb; ++j) {
        const int buf = j & 1;
        float dc, sigma2, alpha, ajc;
        read_step(smem, buf, j, c, dc, sigma2, alpha, ajc);
        const Refl R = reflector(alpha, sigma2);
        const float sv = (c < nb && c != j) ? R.sc * (dc - R.beta * ajc) : 0.f;
        if (slot == 0) {
            smem[OFF_SALL + j * PW + c] = sv;
            if (c == 0) {
                smem[OFF_TAU + j] = R.tau;
                d.rdiag[d.c0 + j] = R.beta;
            }
        }
        const float f = R.tau * sv;
        const int jn = j + 1;
        float pacc = 0.f, sg = 0.f, rj = 0.f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int r = slot + NSLOT * i;
            if (r >= j && r < h) {
                const float vr = (r == j) ? 1.f : R.sc * xc[i];
                if (c == j) x[i] = (r == j) ? R.beta : vr;
                else if (c > j) x[i] -= f * vr;
            }
            const float xn = __shfl(x[i], jn, 32);
            if (r >= jn && r < h) {
                pacc += xn * x[i];
                if (r > jn) sg += xn * xn;
            }
            if (r == jn) rj = x[i];
            xc[i] = xn;
        }
        float* pn = smem + OFF_PART + (buf ^ 1) * PART;
        pn[slot * 33 + c] = pacc;
        if (c == 0) pn[slot * 33 + 32] = sg;
        if (slot == (jn & (NSLOT - 1))) smem[OFF_ROWJ + (buf ^ 1) * 32 + c] = rj;
        __syncthreads();
    }

    // explicit V to global and to LDS (rows padded to 32 with zeros)
    float* Vs = smem + OFF_VS;
    const int hpad = (h + 31) & ~31;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int r = slot + NSLOT * i;
        if (r < hpad) {
            float v = 0.f;
            if (r < h && c < nb) v = (r > c) ? x[i] : (r == c ? 1.f : 0.f);
            Vs[r * 33 + c] = v;
            if (r < h) d.V[(int64_t)r * PW + c] = v;
        }
    }
    build_T(smem, nb, tid);
    __syncthreads();
    form_Y(Vs, 33, smem, d.Y, h, tid);
}

__global__ __launch_bounds__(PANEL_THREADS) void panel_global_kernel(const PanelDesc* __restrict__ descs) {
    extern __shared__ float smem[];
    const PanelDesc d = descs[blockIdx.x];
    const int h = d.h, nb = d.nb;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c = lane & 31;
    const int wv = tid >> 6;
    const int slot = wv * 2 + (lane >> 5);
    const int64_t ld = d.ld;
    float* __restrict__ Ap = d.A + (int64_t)d.c0 * ld + d.c0;

    {   // power-of-two scaling, in place
        float mx = 0.f;
        if (c < nb)
            for (int r = slot; r < h; r += NSLOT) mx = fmaxf(mx, fabsf(Ap[r * ld + c]));
        mx = panel_max(mx, smem, lane, wv);
        if (mx > 0.f) {
            int e;
            frexpf(mx, &e);
            if (c < nb)
                for (int r = slot; r < h; r += NSLOT) Ap[r * ld + c] = ldexpf(Ap[r * ld + c], -e);
        }
        __syncthreads();
    }
    {
        float pacc = 0.f, sg = 0.f, rj = 0.f;
        for (int r = slot; r < h; r += NSLOT) {
            const float xv = (c < nb) ? Ap[r * ld + c] : 0.f;
            const float x0 = Ap[r * ld];
            pacc += x0 * xv;
            if (r > 0) sg += x0 * x0;
            if (r == 0) rj = xv;
        }
        smem[OFF_PART + slot * 33 + c] = pacc;
        if (c == 0) smem[OFF_PART + slot * 33 + 32] = sg;
        if (slot == 0) smem[OFF_ROWJ + c] = rj;
    }
    __syncthreads();

    for (int j = 0; j < nb; ++j) {
        const int buf = j & 1;
        float dc, sigma2, alpha, ajc;
        read_step(smem, buf, j, c, dc, sigma2, alpha, ajc);
        const Refl R = reflector(alpha, sigma2);
        const float sv = (c < nb && c != j) ? R.sc * (dc - R.beta * ajc) : 0.f;
        if (slot == 0) {
            smem[OFF_SALL + j * PW + c] = sv;
            if (c == 0) {
                smem[OFF_TAU + j] = R.tau;
                d.rdiag[d.c0 + j] = R.beta;
            }
        }
        const float f = R.tau * sv;
        const int jn = j + 1;
        float pacc = 0.f, sg = 0.f, rj = 0.f;
        const int r0 = j + ((slot - (j & (NSLOT - 1)) + NSLOT) & (NSLOT - 1));
        for (int r = r0; r < h; r += NSLOT) {
            float xv = (c < nb) ? Ap[r * ld + c] : 0.f;
            const float xj = Ap[r * ld + j];
            const float vr = (r == j) ? 1.f : R.sc * xj;
            if (c == j) {
                xv = (r == j) ? R.beta : vr;
                Ap[r * ld + c] = xv;
            } else if (c > j && c < nb) {
                xv -= f * vr;
                Ap[r * ld + c] = xv;
            }
            const float xn = __shfl(xv, jn, 32);
            if (r >= jn) {
                pacc += xn * xv;
                if (r > jn) sg += xn * xn;
            }
            if (r == jn) rj = xv;
        }
        float* pn = smem + OFF_PART + (buf ^ 1) * PART;
        pn[slot * 33 + c] = pacc;
        if (c == 0) pn[slot * 33 + 32] = sg;
        if (slot == (jn & (NSLOT - 1))) smem[OFF_ROWJ + (buf ^ 1) * 32 + c] = rj;
        __syncthreads();
    }

    for (int r = slot; r < h; r += NSLOT) {
        float v = 0.f;
        if (c < nb) v = (r > c) ? Ap[r * ld + c] : (r == c ? 1.f : 0.f);
        d.V[(int64_t)r * PW + c] = v;
    }
    build_T(smem, nb, tid);
    __syncthreads();
    form_Y(d.V, PW, smem, d.Y, h, tid);
}

template <int NR>
hipError_t launch_reg(const PanelDesc* descs, int ndesc, int max_h, hipStream_t stream) {
    const size_t lds = panel_lds_bytes(true, max_h);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&panel_reg_kernel<NR>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(panel_reg_kernel<NR>, dim3(ndesc), dim3(PANEL_THREADS), lds, stream, descs);
    return hipGetLastError();
}

}  // namespace

int panel_rows_class(int h) {
    if (h > PANEL_LDS_MAX_ROWS) return 0;
    int nr = 2;
    while (NSLOT * nr < h) nr *= 2;
    return nr;
}

size_t panel_lds_bytes(bool in_regs, int max_h) {
    const size_t fixed = (size_t)OFF_VS * sizeof(float);
    const size_t hpad = (size_t)((max_h + 31) & ~31);
    return fixed + (in_regs ? hpad * 33 * sizeof(float) : 0);
}

hipError_t launch_panel(int rows_class, const PanelDesc* descs, int ndesc, int max_h,
                        hipStream_t stream) {
    if (ndesc <= 0) return hipSuccess;
    switch (rows_class) {
        case 2: return launch_reg<2>(descs, ndesc, max_h, stream);
        case 4: return launch_reg<4>(descs, ndesc, max_h, stream);
        case 8: return launch_reg<8>(descs, ndesc, max_h, stream);
        case 16: return launch_reg<16>(descs, ndesc, max_h, stream);
        case 32: return launch_reg<32>(descs, ndesc, max_h, stream);
        case 64: return launch_reg<64>(descs, ndesc, max_h, stream);
        default: break;
    }
    const size_t lds = panel_lds_bytes(false, max_h);
    hipLaunchKernelGGL(panel_global_kernel, dim3(ndesc), dim3(PANEL_THREADS), lds, stream, descs);
    return hipGetLastError();
}

}  // namespace s4
