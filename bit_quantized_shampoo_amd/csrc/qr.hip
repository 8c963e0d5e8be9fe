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
// beta = -sign(alpha) sqrt(d_j), tau = (beta - alpha) / beta,
// v = [1, x_{j+1..} / (alpha - beta)], and
// s_c = v^T A[:, c] = (d_c - beta A[j][c]) / (alpha - beta); a column that is zero
// below the diagonal (d_j == alpha^2 exactly) gives H = I.  beta, tau and v
// involve no cancellation (alpha and beta have opposite signs), so the norm needs
// no separate sum of squares.  One pass applies H_j to the later columns and, in
// the same sweep, accumulates the next column's d_c; the two half-waves of a wave
// combine with one cross-half lane swap, the 8 wave partials meet in LDS
// (column-major, double-buffered by step parity: two 16-byte reads per sum) and
// every thread derives the reflector's scalars itself.  After the update, lane j+1
// of each half-wave publishes its column for the half-wave's rows with 16-byte LDS
// stores and the half-wave reads them back as same-address 16-byte loads (four rows
// per LDS operation, ordered within the wave without a barrier).  The s_c (c < j) of every step are
// kept, and at the end one wave builds T row by row (T[c][j] =
// -tau_j sum_{c <= l < j} T[c][l] s_l, T[j][j] = tau_j) and the workgroup forms
// Y = V T with v_mfma_f32_32x32x2_f32.
//
// The panel is first scaled by a power of two so that its largest entry is in
// [0.5, 1): squares can neither overflow nor (for entries that matter) underflow,
// and V, tau and the signs of R are unchanged by the exact scaling.
#include "kernels.hpp"

namespace s4 {

namespace {

constexpr int NSLOT = PANEL_THREADS / 32;   // row slots (half-waves)
constexpr int NWAVE = PANEL_THREADS / 64;
constexpr int PW = 32;                       // panel width
constexpr int PART = PW * NWAVE;             // one partials buffer: [32 columns][NWAVE]

// LDS layout (floats)
constexpr int OFF_PART = 0;                      // [2][32][NWAVE]
constexpr int OFF_ROWJ = OFF_PART + 2 * PART;    // [2][32]
constexpr int OFF_SALL = OFF_ROWJ + 64;          // [32][32] s vector of step j
constexpr int OFF_TAU = OFF_SALL + PW * PW;      // [32]
constexpr int OFF_T = OFF_TAU + PW;              // [32][33]
constexpr int OFF_RED = OFF_T + PW * 33;         // [NWAVE]
constexpr int OFF_RD = OFF_RED + NWAVE;          // [32] R diagonal (written out after the loop)
constexpr int OFF_COL = ((OFF_RD + PW + 3) / 4) * 4;  // [NSLOT][64] column j+1 of each half-wave's rows
constexpr int OFF_VS = OFF_COL + NSLOT * 64;     // [hpad][33] V staging (register variant)
static_assert(NWAVE == 8, "partials are read as two 16-byte vectors");

struct Refl {
    float tau, beta, sc;
};

// Reflector of column j from alpha = A[j][j] and d = sum_{r >= j} A[r][j]^2.  The
// scalars sit on the critical path of every step, so they use the hardware square
// root and reciprocal (about 1 ulp): Householder QR is backward stable with any
// such rounding; only the codec needs correctly rounded division.
__device__ __forceinline__ Refl reflector(float alpha, float d) {
    Refl s;
    if (d == alpha * alpha) {          // nothing below the diagonal: H = I
        s.tau = 0.f; s.beta = alpha; s.sc = 0.f;
    } else {
        const float nrm = __builtin_amdgcn_sqrtf(d);
        s.beta = (alpha >= 0.f) ? -nrm : nrm;
        const float rb = __builtin_amdgcn_rcpf(s.beta);
        s.tau = (s.beta - alpha) * rb;
        s.sc = __builtin_amdgcn_rcpf(alpha - s.beta);
    }
    return s;
}

__device__ __forceinline__ float sum_partials(const float* p) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(p);
    const floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
    return ((a[0] + a[1]) + (a[2] + a[3])) + ((b[0] + b[1]) + (b[2] + b[3]));
}

// Combined partials of step `buf` for column col, and row j's entry in that column.
__device__ __forceinline__ float read_d(const float* smem, int buf, int col) {
    return sum_partials(smem + OFF_PART + buf * PART + col * NWAVE);
}
__device__ __forceinline__ float read_row(const float* smem, int buf, int col) {
    return smem[OFF_ROWJ + buf * 32 + col];
}

// Store this wave's partial d_c for the step after: the two half-waves (same
// columns, different rows) are added with one cross-half lane swap (a VALU op).
__device__ __forceinline__ void write_partial(float* smem, int buf, int c, int lane, int wv, float pacc) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pacc), __float_as_uint(pacc), false, false);
    const float other = __uint_as_float(lane < 32 ? sw[1] : sw[0]);
    if (lane < 32) smem[OFF_PART + buf * PART + c * NWAVE + wv] = pacc + other;
}

__device__ __forceinline__ float panel_max(float mx, float* smem, int lane, int wv) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) smem[OFF_RED + wv] = mx;
    __syncthreads();
    float m = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) m = fmaxf(m, smem[OFF_RED + w]);
    return m;
}

// T (upper triangular, nb x nb) from the kept s vectors and taus: one lane per row.
// Row c has zeros left of the diagonal, so T[c][j] = -tau_j sum_{l < j} T[c][l] s_l
// for c < j needs no lower bound on l, and the same sum is 0 for c > j.
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
                const float* sj = smem + OFF_SALL + j * PW;
                float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int l = 0; l < j; ++l) acc[l & 3] = fmaf(trow[l], sj[l], acc[l & 3]);
                trow[j] = (c == j) ? tj : -tj * ((acc[0] + acc[1]) + (acc[2] + acc[3]));
            }
        }
#pragma unroll
        for (int l = 0; l < PW; ++l) smem[OFF_T + c * 33 + l] = trow[l];
    }
}

// Y = V T for rows [0, h): V rows come from `vsrc` (pitch vpitch floats), T from LDS,
// Y rows have pitch ypitch.
__device__ __forceinline__ void form_Y(const float* vsrc, int64_t vpitch, const float* smem, float* Y,
                                       int64_t ypitch, int h, int tid) {
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
            const int rc = row < h ? row : h - 1;
            const uint32_t m = row < h ? 0xffffffffu : 0u;
            const float a = __uint_as_float(__float_as_uint(vsrc[(int64_t)rc * vpitch + k]) & m);
            const float b = smem[OFF_T + k * 33 + l32];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int orow = q * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
            if (orow < h) Y[(int64_t)orow * ypitch + l32] = acc[r];
        }
    }
}

// The zrows rows of V and Y above the panel (inside a wider block of reflectors whose
// earlier panels start higher) are zero.
__device__ __forceinline__ void zero_above(const PanelDesc& d, int tid) {
    for (int e = tid; e < d.zrows * PW; e += PANEL_THREADS) {
        const int64_t off = (int64_t)(e / PW) * d.vld + (e % PW);
        d.V[off] = 0.f;
        d.Y[off] = 0.f;
    }
}

// Broadcast of lane `src` of this lane's 32-lane half to every lane of the half.
__device__ __forceinline__ float half_bcast(float v, int byte_addr) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(byte_addr, __float_as_int(v)));
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
    const int half_base = (lane & 32) * 4;        // byte address of lane 0 of this half
    const float* __restrict__ Ap = d.A + (int64_t)d.c0 * d.ld + d.c0;

    // Rows beyond h and columns beyond nb are zero: they stay zero under every update
    // and add nothing to any dot, so only the first row groups (r <= 32, where r may
    // equal j or j+1 or lie above the diagonal) need row tests.
    // All NR loads are issued before any is used: the address is clamped into the panel
    // and the value masked with an AND (a select on the loaded value would become a
    // branch around each load, with a wait for it inside).
    float x[NR], xc[NR];
    {
        const int cc = c < nb ? c : nb - 1;
        const uint32_t cmask = c < nb ? 0xffffffffu : 0u;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int r = slot + NSLOT * i;
            const int rr = r < h ? r : h - 1;
            x[i] = Ap[(int64_t)rr * d.ld + cc];
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const uint32_t m = (slot + NSLOT * i < h) ? cmask : 0u;
            x[i] = __uint_as_float(__float_as_uint(x[i]) & m);
        }
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
    {   // dots for column 0
        float pacc = 0.f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            xc[i] = half_bcast(x[i], half_base);
            pacc = fmaf(xc[i], x[i], pacc);
        }
        write_partial(smem, 0, c, lane, wv, pacc);
        if (slot == 0) smem[OFF_ROWJ + c] = x[0];
    }
    __syncthreads();

    // column j+1 of this half-wave's rows, published by its lane j+1 (same wave: no barrier)
    float* colbuf = smem + OFF_COL + slot * 64;
    for (int j = 0; j < nb; ++j) {
        const int buf = j & 1;
        const int jn = j + 1;
        const float dc = read_d(smem, buf, c);
        const float dj = read_d(smem, buf, j);
        const float alpha = read_row(smem, buf, j);
        const float ajc = read_row(smem, buf, c);
        const Refl R = reflector(alpha, dj);
        const float sv = (c < nb && c != j) ? R.sc * (dc - R.beta * ajc) : 0.f;
        if (slot == 0) {
            smem[OFF_SALL + j * PW + c] = sv;
            if (c == 0) {
                smem[OFF_TAU + j] = R.tau;
                smem[OFF_RD + j] = R.beta;   // no global store inside the loop
            }
        }
        const float f = R.tau * sv;                      // 0 for columns c < j
        // rows below j: x <- x + coef * xc.  Lane j stores v = sc * x; its xc equals its
        // own x, so x + (sc - 1) x is that value with one fused multiply-add.
        const float coef = (c == j) ? R.sc - 1.f : ((c > j) ? -f * R.sc : 0.f);
        // row j: lane j stores beta, later columns subtract f (v_j = 1)
        const float diag_val = (c == j) ? R.beta : 0.f;
        const float diag_keep = (c == j) ? 0.f : 1.f;
        const float diag_sub = (c > j) ? f : 0.f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const float xv = x[i];
            float nx = fmaf(coef, xc[i], xv);
            if (NSLOT * i < PW) {
                const int r = slot + NSLOT * i;
                const float dgv = fmaf(diag_keep, xv, diag_val) - diag_sub;
                nx = (r < j) ? xv : ((r == j) ? dgv : nx);
            }
            x[i] = nx;
        }
        if (c == jn) {
            if constexpr (NR % 4 == 0) {
#pragma unroll
                for (int q = 0; q < NR / 4; ++q) {
                    const floatx4 v = {x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
                    *reinterpret_cast<floatx4*>(colbuf + 4 * q) = v;
                }
            } else {
#pragma unroll
                for (int i = 0; i < NR; ++i) colbuf[i] = x[i];
            }
        }
        // lanes of one wave exchange through LDS: order the stores before the loads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float pacc = 0.f, rj = 0.f;
#pragma unroll
        for (int q = 0; q < (NR + 3) / 4; ++q) {
            float xn4[4];
            if constexpr (NR % 4 == 0) {
                const floatx4 v = *reinterpret_cast<const floatx4*>(colbuf + 4 * q);
                xn4[0] = v[0]; xn4[1] = v[1]; xn4[2] = v[2]; xn4[3] = v[3];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) xn4[e] = (4 * q + e < NR) ? colbuf[4 * q + e] : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * q + e;
                if (i < NR) {
                    const float xn = xn4[e];
                    if (NSLOT * i <= PW) {
                        const int r = slot + NSLOT * i;
                        pacc += (r >= jn) ? xn * x[i] : 0.f;
                        rj = (r == jn) ? x[i] : rj;
                    } else {
                        pacc = fmaf(xn, x[i], pacc);
                    }
                    xc[i] = xn;
                }
            }
        }
        write_partial(smem, buf ^ 1, c, lane, wv, pacc);
        if (slot == (jn & (NSLOT - 1))) smem[OFF_ROWJ + (buf ^ 1) * 32 + c] = rj;
        __syncthreads();
    }

    if (tid < nb) d.rdiag[d.c0 + tid] = smem[OFF_RD + tid];
    // explicit V to global and to LDS (rows padded to 32 with zeros)
    float* Vs = smem + OFF_VS;
    float* Vt = d.V + (int64_t)d.zrows * d.vld;
    float* Yt = d.Y + (int64_t)d.zrows * d.vld;
    const int hpad = (h + 31) & ~31;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int r = slot + NSLOT * i;
        if (r < hpad) {
            float v = 0.f;
            if (r < h && c < nb) v = (r > c) ? x[i] : (r == c ? 1.f : 0.f);
            Vs[r * 33 + c] = v;
            if (r < h) Vt[(int64_t)r * d.vld + c] = v;
        }
    }
    build_T(smem, nb, tid);
    zero_above(d, tid);
    __syncthreads();
    form_Y(Vs, 33, smem, Yt, d.vld, h, tid);
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
        float pacc = 0.f, rj = 0.f;
        for (int r = slot; r < h; r += NSLOT) {
            const float xv = (c < nb) ? Ap[r * ld + c] : 0.f;
            const float x0 = Ap[r * ld];
            pacc += x0 * xv;
            if (r == 0) rj = xv;
        }
        write_partial(smem, 0, c, lane, wv, pacc);
        if (slot == 0) smem[OFF_ROWJ + c] = rj;
    }
    __syncthreads();

    for (int j = 0; j < nb; ++j) {
        const int buf = j & 1;
        const float dc = read_d(smem, buf, c);
        const float dj = read_d(smem, buf, j);
        const float alpha = read_row(smem, buf, j);
        const float ajc = read_row(smem, buf, c);
        const Refl R = reflector(alpha, dj);
        const float sv = (c < nb && c != j) ? R.sc * (dc - R.beta * ajc) : 0.f;
        if (slot == 0) {
            smem[OFF_SALL + j * PW + c] = sv;
            if (c == 0) {
                smem[OFF_TAU + j] = R.tau;
                smem[OFF_RD + j] = R.beta;   // no global store inside the loop
            }
        }
        const float f = R.tau * sv;
        const int jn = j + 1;
        float pacc = 0.f, rj = 0.f;
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
            if (r >= jn) pacc += xn * xv;
            if (r == jn) rj = xv;
        }
        write_partial(smem, buf ^ 1, c, lane, wv, pacc);
        if (slot == (jn & (NSLOT - 1))) smem[OFF_ROWJ + (buf ^ 1) * 32 + c] = rj;
        __syncthreads();
    }

    if (tid < nb) d.rdiag[d.c0 + tid] = smem[OFF_RD + tid];
    float* Vt = d.V + (int64_t)d.zrows * d.vld;
    float* Yt = d.Y + (int64_t)d.zrows * d.vld;
    for (int r = slot; r < h; r += NSLOT) {
        float v = 0.f;
        if (c < nb) v = (r > c) ? Ap[r * ld + c] : (r == c ? 1.f : 0.f);
        Vt[(int64_t)r * d.vld + c] = v;
    }
    build_T(smem, nb, tid);
    zero_above(d, tid);
    __syncthreads();
    form_Y(Vt, d.vld, smem, Yt, d.vld, h, tid);
}

template <int NR>
hipError_t launch_reg(const PanelDesc* descs, int ndesc, int max_h, hipStream_t stream) {
    // the dynamic-LDS limit is raised once per instantiation (to the largest panel it serves)
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&panel_reg_kernel<NR>), hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)panel_lds_bytes(true, NSLOT * NR < PANEL_LDS_MAX_ROWS ? NSLOT * NR : PANEL_LDS_MAX_ROWS));
    if (attr != hipSuccess) return attr;
    const size_t lds = panel_lds_bytes(true, max_h);
    S4_LAUNCH(panel_reg_kernel<NR>, dim3(ndesc), dim3(PANEL_THREADS), lds, stream, descs);
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
    S4_LAUNCH(panel_global_kernel, dim3(ndesc), dim3(PANEL_THREADS), lds, stream, descs);
    return hipGetLastError();
}

}  // namespace s4
