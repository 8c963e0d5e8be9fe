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
// one partials buffer: [32 columns][PSTR], NWAVE used; the 12-float column pitch keeps the
// two 16-byte reads of 8 consecutive lanes' columns on distinct banks
constexpr int PSTR = 12;
constexpr int PART = PW * PSTR;

// LDS layout (floats)
constexpr int OFF_PART = 0;                      // [2][32][PSTR]
constexpr int OFF_ROWJ = OFF_PART + 2 * PART;    // [2][32]
constexpr int OFF_SALL = OFF_ROWJ + 64;          // [32 columns][33] s_j[c] of step j at c * 33 + j
constexpr int OFF_TAU = OFF_SALL + PW * 33;      // [32]
constexpr int OFF_T = OFF_TAU + PW;              // [32][33]
constexpr int OFF_RED = OFF_T + PW * 33;         // [NWAVE]
constexpr int OFF_RD = OFF_RED + NWAVE;          // [32] R diagonal (written out after the loop)
// Column j+1 of each half-wave's rows: the two half-waves of a wave read their slots in
// the same instruction, so the slot pitch is offset by 4 banks from a multiple of the bank
// count (64 + 4 floats): the two 16-byte broadcasts hit different banks.
constexpr int COL_PITCH = 68;
// Rows per lane (one-column count) from which panels take the two-column layout: below
// it the one-column loop is faster (measured per register class on 1024-sized blocks).
constexpr int kTwoColMinNR = 24;
// Two-column layout (panels of more than 320 rows): row group G's slice of the pivot column
// at G * COL2_PITCH; the four row groups of a wave read theirs in one instruction, so the
// pitch sits 4 banks off a multiple of the bank count.
constexpr int NGRP = PANEL_THREADS / 16;     // row groups of 16 lanes
constexpr int COL2_PITCH = 36;
constexpr int COL_AREA = NSLOT * COL_PITCH > NGRP * COL2_PITCH ? NSLOT * COL_PITCH : NGRP * COL2_PITCH;
constexpr int OFF_COL = ((OFF_RD + PW + 3) / 4) * 4;  // [NSLOT][COL_PITCH] or [NGRP][COL2_PITCH]
constexpr int OFF_VS = OFF_COL + COL_AREA;  // [rows][33] V staging / layout transpose (register variant)
constexpr int OFF_VS_T12 = OFF_COL;              // [16][16] scratch of build_T (after the loop)
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
    return sum_partials(smem + OFF_PART + buf * PART + col * PSTR);
}
__device__ __forceinline__ float read_row(const float* smem, int buf, int col) {
    return smem[OFF_ROWJ + buf * 32 + col];
}

// Store this wave's partial d_c for the step after: the two half-waves (same
// columns, different rows) are added with one cross-half lane swap (a VALU op).
__device__ __forceinline__ void write_partial(float* smem, int buf, int c, int lane, int wv, float pacc) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pacc), __float_as_uint(pacc), false, false);
    const float other = __uint_as_float(lane < 32 ? sw[1] : sw[0]);
    if (lane < 32) smem[OFF_PART + buf * PART + c * PSTR + wv] = pacc + other;
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

// T (upper triangular, nb x nb) from the kept s vectors and taus, into LDS at OFF_T (pitch
// 33), by the whole workgroup (two barriers inside).  T[c][j] = -tau_j sum_{c <= l < j} T[c][l]
// s_j[l], T[j][j] = tau_j, with s_j[l] = v_j^T v_l at smem[OFF_SALL + l * 33 + j].  Blocked in
// halves: the two diagonal 16 x 16 blocks run in parallel (one lane per row, right-looking:
// once T[c][l] is known it is added into the running sums of every later column, so each step's
// dependent work is one multiply and one fused multiply-add), then T12 = -T11 (V1^T V2) T22.
// Entries of s for steps >= nb were never written: in the recurrence they only reach running
// sums of columns >= nb, whose T entries are selected to zero, and in the off-diagonal product
// they are masked.
__device__ __forceinline__ void build_T_diag(float* smem, int nb, int tid) {
    const int lane = tid & 63;
    if (tid < 64 && (lane & 31) < 16) {
        const int blk = lane >> 5, c = lane & 15;
        const int b0 = 16 * blk, row = b0 + c;
        float acc[16], trow[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#pragma unroll
        for (int ll = 0; ll < 16; ++ll) {
            const int l = b0 + ll;
            const float tl = smem[OFF_TAU + l];
            float t = (c == ll) ? tl : ((c < ll) ? -tl * acc[ll] : 0.f);
            t = (l < nb) ? t : 0.f;
            trow[ll] = t;
            const float* sl = smem + OFF_SALL + l * 33 + b0;
#pragma unroll
            for (int j = ll + 1; j < 16; ++j) acc[j] = fmaf(t, sl[j], acc[j]);
        }
#pragma unroll
        for (int ll = 0; ll < 16; ++ll) {
            smem[OFF_T + row * 33 + b0 + ll] = trow[ll];
            if (blk == 1) smem[OFF_T + row * 33 + ll] = 0.f;        // below the diagonal blocks
        }
    }
}

// The off-diagonal block, after build_T_diag and a barrier (one more barrier inside).
__device__ __forceinline__ void build_T_offdiag(float* smem, int nb, int tid) {
    // X = S12 T22 (16 x 16, kept in the T12 slot's registers): S12[l][m] = s_{16+m}[l]
    float x = 0.f;
    const int xr = (tid >> 4) & 15, xc = tid & 15;
    if (tid < 256) {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const uint32_t ok = 16 + m < nb ? 0xffffffffu : 0u;
            const float s12 = __uint_as_float(__float_as_uint(smem[OFF_SALL + xr * 33 + 16 + m]) & ok);
            x = fmaf(s12, smem[OFF_T + (16 + m) * 33 + 16 + xc], x);
        }
        smem[OFF_VS_T12 + xr * 16 + xc] = x;
    }
    __syncthreads();
    if (tid < 256) {   // T12 = -T11 X
        float t12 = 0.f;
#pragma unroll
        for (int l = 0; l < 16; ++l) t12 = fmaf(smem[OFF_T + xr * 33 + l], smem[OFF_VS_T12 + l * 16 + xc], t12);
        smem[OFF_T + xr * 33 + 16 + xc] = -t12;
    }
}

__device__ __forceinline__ void build_T(float* smem, int nb, int tid) {
    build_T_diag(smem, nb, tid);
    __syncthreads();
    build_T_offdiag(smem, nb, tid);
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

// ---- Compact-WY application of a reflector block on the matrix cores -------------------
// A block of nb <= 32 reflectors (explicit V: h rows, 32 columns of which those beyond nb
// are zero, pitch vld; T: 32 x 32 upper triangular) multiplies to I - V T V^T.  The fused QR
// step applies it from the left to columns of P (M <- M - V (T^T (V^T M)): the trailing
// update) and from the right to rows of Q (M <- M - ((M V) T) V^T: the forward accumulation
// of Q).  The long products are 32 x 32 x K contractions on v_mfma_f32_32x32x2_f32: the 8
// waves split K and add their 32 x 32 partial results in LDS in a fixed order; T is applied
// to the 32 x 32 result on the vector units; then each wave updates its share of 32-row (or
// 32-column) blocks.  Inside a 32-deep contraction, lane half hh takes k = ks + 16 hh, so a
// lane reads 16 consecutive floats of a V row.

constexpr int WY_PART = 8 * 32 * 36;   // floats of per-wave partial products (or V tiles) in LDS

__device__ __forceinline__ int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

__device__ __forceinline__ float masked(float v, uint32_t m) { return __uint_as_float(__float_as_uint(v) & m); }

// Operands of one 32-deep block of a contraction, held while the next block's loads fly.
struct WyBuf {
    float a[16], b[16];
};

// Items first, first + 8, ... < n of one wave, two deep: the loads of item i + 8 are issued
// before the matrix-core work of item i.
template <class Load, class Use>
__device__ __forceinline__ void wy_pipeline(int first, int n, Load load, Use use) {
    WyBuf b0, b1;
    int it = first;
    if (it < n) load(it, b0);
    for (; it < n; it += 16) {
        const bool more = it + 8 < n;
        if (more) load(it + 8, b1);
        use(it, b0);
        if (more) {
            if (it + 16 < n) load(it + 16, b0);
            use(it + 8, b1);
        }
    }
}

// out[m * 32 + n] = sum over the 8 waves of their accumulators (fixed order).
__device__ __forceinline__ void wy_reduce(const floatx16& acc, float* part, float* out, int tid) {
    const int lane = tid & 63, wv = tid >> 6, l32 = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int r = 0; r < 16; ++r) part[wv * 1024 + acc_row(r, hh) * 32 + l32] = acc[r];
    __syncthreads();
    for (int e = tid; e < 1024; e += PANEL_THREADS) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) s += part[w * 1024 + e];
        out[e] = s;
    }
    __syncthreads();
}

// Sixteen consecutive floats of a V row (16-byte aligned: V rows have pitch 32).
__device__ __forceinline__ void load_vrow16(const float* p, float (&v)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const floatx4 t = ldg(reinterpret_cast<const floatx4*>(p) + q);
        v[4 * q] = t[0]; v[4 * q + 1] = t[1]; v[4 * q + 2] = t[2]; v[4 * q + 3] = t[3];
    }
}

// W[i][c] = sum_{r < h} Y[r][i] M[r][c] for c < ncols (W row-major 32 x 32 in LDS); Y is a
// 32-column block (V in the fused step).
// Wave w takes the 32-row blocks w, w + 8, ...; in a block, lane half hh reads rows
// ks + 16 hh (one coalesced row per half-wave and step).
__device__ __forceinline__ void wy_left_product(const float* __restrict__ Y, int64_t vld, const float* __restrict__ M,
                                int64_t ld, int h, int ncols, float* part, float* W, int tid) {
    const int lane = tid & 63, wv = tid >> 6, l32 = lane & 31, hh = lane >> 5;
    const int cc = l32 < ncols ? l32 : ncols - 1;
    const uint32_t cm = l32 < ncols ? 0xffffffffu : 0u;
    floatx16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    auto load = [&](int bk, WyBuf& B) {
        const int rb = 32 * bk + 16 * hh;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const int rr = rb + ks < h ? rb + ks : h - 1;
            B.a[ks] = ldg(Y + (int64_t)rr * vld + l32);
            B.b[ks] = ldg(M + (int64_t)rr * ld + cc);
        }
    };
    auto use = [&](int bk, const WyBuf& B) {
        const int rb = 32 * bk + 16 * hh;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const uint32_t rm = rb + ks < h ? 0xffffffffu : 0u;
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(masked(B.a[ks], rm), masked(B.b[ks], rm & cm), acc, 0, 0, 0);
        }
    };
    wy_pipeline(wv, (h + 31) / 32, load, use);
    wy_reduce(acc, part, W, tid);
}

// M[r][c] -= sum_i V[r][i] W[i][c] for rows r < h and columns c < ncols.
__device__ __forceinline__ void wy_update_rows(const float* __restrict__ V, int64_t vld, float* M, int64_t ld,
                                               int h, int ncols, const float* W, int tid) {
    const int lane = tid & 63, wv = tid >> 6, l32 = lane & 31, hh = lane >> 5;
    const int cc = l32 < ncols ? l32 : ncols - 1;
    float wb[16];                                     // B operand: W[ks + 16 hh][l32]
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) wb[ks] = W[(16 * hh + ks) * 32 + l32];
    auto load = [&](int bk, WyBuf& B) {              // a: the block of M (C operand), b: V row
        const int rb = 32 * bk;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = rb + acc_row(r, hh);
            B.a[r] = ldg(M + (int64_t)(row < h ? row : h - 1) * ld + cc);
        }
        const int vr = rb + l32 < h ? rb + l32 : h - 1;
        load_vrow16(V + (int64_t)vr * vld + 16 * hh, B.b);   // A operand: V[rb + l32][ks + 16 hh]
    };
    auto use = [&](int bk, const WyBuf& B) {
        const int rb = 32 * bk;
        floatx16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = B.a[r];
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(-B.b[ks], wb[ks], acc, 0, 0, 0);
        if (l32 < ncols) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = rb + acc_row(r, hh);
                if (row < h) stg(M + (int64_t)row * ld + l32, acc[r]);
            }
        }
    };
    wy_pipeline(wv, (h + 31) / 32, load, use);
}

// Z[m][i] = sum_{k < h} M[m][k] Y[k][i] for rows m < nrows of M (Z row-major 32 x 32 in LDS);
// Y is a 32-column block (V in the fused step).
// Wave w takes the 32-column chunks w, w + 8, ...
// ident: M is the identity shifted by diag (M[m][k] = [m + diag == k]), not read.
__device__ __forceinline__ void wy_right_product(const float* __restrict__ M, int64_t ld, int nrows, const float* __restrict__ Y,
                                 int64_t vld, int h, float* part, float* Z, int tid, bool ident = false,
                                 int64_t diag = 0) {
    const int lane = tid & 63, wv = tid >> 6, l32 = lane & 31, hh = lane >> 5;
    const int mr = l32 < nrows ? l32 : nrows - 1;
    const uint32_t rmask = l32 < nrows ? 0xffffffffu : 0u;
    // the identity is merged in with a bit mask after an unconditional load (a select
    // on a loaded value would become a branch around the load)
    const uint32_t keep = ident ? 0u : 0xffffffffu;
    floatx16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    auto load = [&](int t, WyBuf& B) {
        const int kb = 32 * t + 16 * hh;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const int k = kb + ks < h ? kb + ks : h - 1;
            const float mv = ldg(M + (int64_t)mr * ld + k);    // A operand: M[l32][k]
            const uint32_t iv = (mr + diag == k) ? 0x3f800000u : 0u;
            B.a[ks] = __uint_as_float((__float_as_uint(mv) & keep) | (iv & ~keep));
            B.b[ks] = ldg(Y + (int64_t)k * vld + l32);  // B operand: Y[k][l32]
        }
    };
    auto use = [&](int t, const WyBuf& B) {
        const int kb = 32 * t + 16 * hh;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const uint32_t km = kb + ks < h ? 0xffffffffu : 0u;
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(masked(B.a[ks], km & rmask), masked(B.b[ks], km), acc, 0, 0, 0);
        }
    };
    wy_pipeline(wv, (h + 31) / 32, load, use);
    wy_reduce(acc, part, Z, tid);
}

// M[m][c] -= sum_i Z[m][i] V[c][i] for rows m < nrows and columns c < h.
__device__ __forceinline__ void wy_update_cols(float* M, int64_t ld, int nrows, const float* __restrict__ V, int64_t vld, int h,
                               const float* Z, int tid, bool ident = false, int64_t diag = 0) {
    const int lane = tid & 63, wv = tid >> 6, l32 = lane & 31, hh = lane >> 5;
    float za[16];                                     // A operand: -Z[l32][ks + 16 hh]
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) za[ks] = -Z[l32 * 32 + 16 * hh + ks];
    const uint32_t keep = ident ? 0u : 0xffffffffu;   // identity merged in after the load
    auto load = [&](int t, WyBuf& B) {               // a: the block of M (C operand), b: V row
        const int col = 32 * t + l32 < h ? 32 * t + l32 : h - 1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = acc_row(r, hh);
            const int rr = row < nrows ? row : nrows - 1;
            const float mv = ldg(M + (int64_t)rr * ld + col);
            const uint32_t iv = (rr + diag == col) ? 0x3f800000u : 0u;
            B.a[r] = __uint_as_float((__float_as_uint(mv) & keep) | (iv & ~keep));
        }
        load_vrow16(V + (int64_t)col * vld + 16 * hh, B.b);  // B operand: V[32 t + l32][ks + 16 hh]
    };
    auto use = [&](int t, const WyBuf& B) {
        const int cb = 32 * t;
        floatx16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = B.a[r];
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(za[ks], B.b[ks], acc, 0, 0, 0);
        if (cb + l32 < h) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = acc_row(r, hh);
                if (row < nrows) stg(M + (int64_t)row * ld + cb + l32, acc[r]);
            }
        }
    };
    wy_pipeline(wv, (h + 31) / 32, load, use);
}

// T (32 x 32, row-major in global memory) into LDS at Tl with pitch 33.
__device__ __forceinline__ void load_T(const float* __restrict__ T, float* Tl, int tid) {
    for (int e = tid; e < PW * PW; e += PANEL_THREADS) Tl[(e >> 5) * 33 + (e & 31)] = ldg(T + e);
}

// X (32 x 32, row-major in LDS) <- T^T X (LEFT) or X T, T in LDS with pitch 33; fixed order.
template <bool LEFT>
__device__ __forceinline__ void wy_apply_t(const float* Tl, float* X, int tid) {
    float o[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int e = tid + u * PANEL_THREADS;
        const int row = e >> 5, col = e & 31;
        float acc = 0.f;
#pragma unroll
        for (int l = 0; l < PW; ++l)
            acc = LEFT ? fmaf(Tl[l * 33 + row], X[l * 32 + col], acc) : fmaf(X[row * 32 + l], Tl[l * 33 + col], acc);
        o[u] = acc;
    }
    __syncthreads();
    X[tid] = o[0];
    X[tid + PANEL_THREADS] = o[1];
    __syncthreads();
}

// Extra arguments of the panel in a fused QR step: the previous panel's block (Vp, Tp, nbp
// reflectors, nbp = 0: none) and where this panel's T goes.
struct PanelExtra {
    const float* Vp;
    const float* Tp;
    float* T;
    int nbp;
};

// The register-resident panel factorization of one workgroup.
// MODE 0: a panel of the blocked / look-ahead QR: writes V and Y = V T.
// MODE 1: a panel of a fused QR step: writes V and T (the consumers apply T themselves).
// MODE 2: as 1, after first applying the previous panel's block I - Vp Tp Vp^T (transposed,
//         from the left) to the panel's columns, in registers.
// Value of the lane in the partner 16-lane row (rows 0-1 and 2-3 pair up), and in the other
// 32-lane half (v_permlane16_swap / v_permlane32_swap of a value with itself).
__device__ __forceinline__ float other_row16(float v, int lane) {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 16) ? sw[0] : sw[1]);
}
__device__ __forceinline__ float other_half32(float v, int lane) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 32) ? sw[0] : sw[1]);
}
// Sum over the four 16-lane rows of a wave, the same value in every lane.
__device__ __forceinline__ float rows4_sum(float v, int lane) {
    const float a = v + other_row16(v, lane);
    return a + other_half32(a, lane);
}

// The reflector loop and the outputs of panels with more than 320 rows (24 or more rows per
// lane in the one-column layout), two columns per lane.
// With one column per lane, step j's pivot column lives in one lane of each half-wave,
// which stores NR values for its half-wave to read back: NR/4 16-byte LDS stores per wave
// and step with two active lanes each, and those stores (not the reads, which are
// same-address broadcasts) are what a step of a tall panel waits on.  Here lane bits 0..3
// pick the column pair (c16, c16 + 16) and bits 4..5 the row group: row group
// G = 4 wv + g owns rows G + 32 i, so the pivot column of a row group still sits in one
// lane, but the four row groups of a wave store their NR/2 values in the same instructions
// (half the stores).  The panel is handed over from the one-column layout of the load and
// the previous block's application through LDS (rows x 33 floats).
template <int NR, int MODE>
__device__ __forceinline__ void panel_two_cols(const PanelDesc& d, const PanelExtra& ex, float* smem,
                                               const float (&x)[NR]) {
    static_assert(NR % 2 == 0, "two rows of the one-column layout per row of the two-column one");
    constexpr int NR2 = NR / 2;
    const int h = d.h, nb = d.nb;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int c = lane & 31;
    const int slot = wv * 2 + (lane >> 5);
    const int c16 = lane & 15;
    const int g = lane >> 4;
    const int G = 4 * wv + g;
    // hand-over: rows slot + 16 i of column c -> LDS -> rows G + 32 i of columns c16, c16 + 16
    float* tr = smem + OFF_VS;
#pragma unroll
    for (int i = 0; i < NR; ++i) tr[(slot + NSLOT * i) * 33 + c] = x[i];
    __syncthreads();
    float y[2][NR2], yc[NR2];
#pragma unroll
    for (int i = 0; i < NR2; ++i) {
        const float* row = tr + (G + NGRP * i) * 33;
        y[0][i] = row[c16];
        y[1][i] = row[c16 + 16];
        yc[i] = row[0];
    }
    {   // dots with column 0, row 0 of every column
        float pacc[2] = {0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NR2; ++i)
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) pacc[sl] = fmaf(yc[i], y[sl][i], pacc[sl]);
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            const float t = rows4_sum(pacc[sl], lane);
            if (g == 0) smem[OFF_PART + (c16 + 16 * sl) * PSTR + wv] = t;
        }
        if (G == 0) {
            smem[OFF_ROWJ + c16] = y[0][0];
            smem[OFF_ROWJ + c16 + 16] = y[1][0];
        }
    }
    __syncthreads();

    float* colb = smem + OFF_COL + G * COL2_PITCH;
    for (int j = 0; j < nb; ++j) {
        const int buf = j & 1;
        const int jn = j + 1;
        // even row groups sum column c16's partials, odd ones column c16 + 16's; lane j
        // (row group j >> 4, c16 = j & 15) holds the pivot column's
        const int sr = g & 1;
        const float dm = read_d(smem, buf, c16 + 16 * sr);
        const float am = read_row(smem, buf, c16 + 16 * sr);
        const float dmo = other_row16(dm, lane);
        const float amo = other_row16(am, lane);
        const float dcs[2] = {sr ? dmo : dm, sr ? dm : dmo};
        const float acs[2] = {sr ? amo : am, sr ? am : amo};
        const float dj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dm), j));
        const float alpha = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(am), j));
        const Refl R = reflector(alpha, dj);
        float sv[2], coef[2], dval[2], dkeep[2], dsub[2];
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            const int cs = c16 + 16 * sl;
            sv[sl] = (cs < nb && cs != j) ? R.sc * (dcs[sl] - R.beta * acs[sl]) : 0.f;
            const float f = R.tau * sv[sl];
            coef[sl] = (cs == j) ? R.sc - 1.f : ((cs > j) ? -f * R.sc : 0.f);
            dval[sl] = (cs == j) ? R.beta : 0.f;
            dkeep[sl] = (cs == j) ? 0.f : 1.f;
            dsub[sl] = (cs > j) ? f : 0.f;
        }
        if (G == 0) {
            smem[OFF_SALL + c16 * 33 + j] = sv[0];
            smem[OFF_SALL + (c16 + 16) * 33 + j] = sv[1];
            if (c16 == 0) {
                smem[OFF_TAU + j] = R.tau;
                smem[OFF_RD + j] = R.beta;
            }
        }
        // update (rows below j: y + coef yc; row j: the pivot lane stores beta, later columns
        // subtract f); columns 0..15 are all final once j > 15
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            if (sl == 0 && j > 15) continue;
#pragma unroll
            for (int i = 0; i < NR2; ++i) {
                const float xv = y[sl][i];
                float nx = fmaf(coef[sl], yc[i], xv);
                if (i == 0) {
                    const float dgv = fmaf(dkeep[sl], xv, dval[sl]) - dsub[sl];
                    nx = (G < j) ? xv : ((G == j) ? dgv : nx);
                }
                y[sl][i] = nx;
            }
        }
        // column jn of this row group's rows, from its lane (c16 = jn & 15)
        if (jn < nb && c16 == (jn & 15)) {
            const int sn = jn >> 4;
            float vn[NR2];
#pragma unroll
            for (int i = 0; i < NR2; ++i) vn[i] = sn ? y[1][i] : y[0][i];
            if constexpr (NR2 % 4 == 0) {
#pragma unroll
                for (int q = 0; q < NR2 / 4; ++q) {
                    const floatx4 v = {vn[4 * q], vn[4 * q + 1], vn[4 * q + 2], vn[4 * q + 3]};
                    *reinterpret_cast<floatx4*>(colb + 4 * q) = v;
                }
            } else {
#pragma unroll
                for (int i = 0; i < NR2; ++i) colb[i] = vn[i];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float xn[NR2];
        if constexpr (NR2 % 4 == 0) {
#pragma unroll
            for (int q = 0; q < NR2 / 4; ++q) {
                const floatx4 v = *reinterpret_cast<const floatx4*>(colb + 4 * q);
                xn[4 * q] = v[0]; xn[4 * q + 1] = v[1]; xn[4 * q + 2] = v[2]; xn[4 * q + 3] = v[3];
            }
        } else {
#pragma unroll
            for (int i = 0; i < NR2; ++i) xn[i] = colb[i];
        }
        float pacc[2] = {0.f, 0.f}, rj[2] = {0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NR2; ++i) {
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                if (i == 0) {   // rows 0..31: only rows >= jn count
                    pacc[sl] += (G >= jn) ? xn[0] * y[sl][0] : 0.f;
                    rj[sl] = (G == jn) ? y[sl][0] : rj[sl];
                } else {
                    pacc[sl] = fmaf(xn[i], y[sl][i], pacc[sl]);
                }
            }
            yc[i] = xn[i];
        }
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            const float t = rows4_sum(pacc[sl], lane);
            if (g == 0) smem[OFF_PART + (buf ^ 1) * PART + (c16 + 16 * sl) * PSTR + wv] = t;
        }
        if (G == jn) {
            smem[OFF_ROWJ + (buf ^ 1) * 32 + c16] = rj[0];
            smem[OFF_ROWJ + (buf ^ 1) * 32 + c16 + 16] = rj[1];
        }
        __syncthreads();
    }

    if (tid < nb) d.rdiag[d.c0 + tid] = smem[OFF_RD + tid];
    float* Vt = d.V + (int64_t)d.zrows * d.vld;
    auto vval = [&](int sl, int i) {
        const int r = G + NGRP * i, cs = c16 + 16 * sl;
        float v = 0.f;
        if (r < h && cs < nb) v = (r > cs) ? y[sl][i] : (r == cs ? 1.f : 0.f);
        return v;
    };
    if constexpr (MODE == 0) {
        // explicit V to global and to LDS (rows padded to 32 with zeros), then Y = V T
        float* Vs = smem + OFF_VS;
        float* Yt = d.Y + (int64_t)d.zrows * d.vld;
        const int hpad = (h + 31) & ~31;
#pragma unroll
        for (int i = 0; i < NR2; ++i) {
            const int r = G + NGRP * i;
            if (r < hpad) {
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) {
                    const float v = vval(sl, i);
                    Vs[r * 33 + c16 + 16 * sl] = v;
                    if (r < h) Vt[(int64_t)r * d.vld + c16 + 16 * sl] = v;
                }
            }
        }
        build_T(smem, nb, tid);
        zero_above(d, tid);
        __syncthreads();
        form_Y(Vs, 33, smem, Yt, d.vld, h, tid);
    } else {
        auto write_v = [&]() {
#pragma unroll
            for (int i = 0; i < NR2; ++i) {
                const int r = G + NGRP * i;
                if (r < h) {
#pragma unroll
                    for (int sl = 0; sl < 2; ++sl) stg(Vt + (int64_t)r * d.vld + c16 + 16 * sl, vval(sl, i));
                }
            }
        };
        if (wv != 0) write_v();
        build_T_diag(smem, nb, tid);
        if (wv == 0) write_v();
        __syncthreads();
        build_T_offdiag(smem, nb, tid);
        __syncthreads();
        for (int e = tid; e < PW * PW; e += PANEL_THREADS) stg(ex.T + e, smem[OFF_T + (e >> 5) * 33 + (e & 31)]);
    }
}

template <int NR, int MODE>
__device__ __forceinline__ void panel_body(const PanelDesc& d, const PanelExtra& ex, float* smem) {
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
    float pa[MODE == 2 ? NR : 1], pa_top[2], pb_top[2];   // MODE 2: operands of the previous block
    {
        const int cc = c < nb ? c : nb - 1;
        const uint32_t cmask = c < nb ? 0xffffffffu : 0u;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int r = slot + NSLOT * i;
            const int rr = r < h ? r : h - 1;
            x[i] = ldg(Ap + (int64_t)rr * d.ld + cc);
        }
        if constexpr (MODE == 2) {
            // the previous block's operands, issued together with the panel's own loads
            const int nbp = ex.nbp;
            const float* Atop = d.A + (int64_t)(d.c0 - nbp) * d.ld + d.c0;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int tr = slot + NSLOT * t;
                const int trc = tr < nbp ? tr : nbp - 1;
                pa_top[t] = ldg(ex.Vp + (int64_t)trc * d.vld + c);
                pb_top[t] = ldg(Atop + (int64_t)trc * d.ld + cc);
            }
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const int r = slot + NSLOT * i;
                const int rr = r < h ? r : h - 1;
                pa[i] = ldg(ex.Vp + (int64_t)(nbp + rr) * d.vld + c);
            }
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const uint32_t m = (slot + NSLOT * i < h) ? cmask : 0u;
            x[i] = __uint_as_float(__float_as_uint(x[i]) & m);
        }
    }
    if constexpr (MODE == 2) {
        // Previous block on this panel's columns: x <- x - Vp (Tp^T (Vp^T A)), where the
        // contraction Vp^T A runs over the block's rows: its nbp rows above the panel and
        // the panel's own rows, which this lane holds in x.  MFMA i of a wave takes the
        // rows of x[i] of its two half-waves, so x[i] itself is the B operand; the update
        // takes x[16 vb .. 16 vb + 15] as its accumulator, the A operand being the V rows
        // that the accumulator layout assigns to each lane.
        const int hh = lane >> 5;
        const int nbp = ex.nbp;
        load_T(ex.Tp, smem + OFF_T, tid);
        const uint32_t cmask = c < nb ? 0xffffffffu : 0u;
        floatx16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t m = slot + NSLOT * t < nbp ? 0xffffffffu : 0u;
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(masked(pa_top[t], m), masked(pb_top[t], m & cmask), acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const uint32_t m = slot + NSLOT * i < h ? 0xffffffffu : 0u;
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(masked(pa[i], m), x[i], acc, 0, 0, 0);
        }
        constexpr int NVB = (NR + 15) / 16;
        // accumulator row m of this lane's A operand: m = c = 8 q + 4 hq + e
        const int q = c >> 3, hq = (c >> 2) & 1, e4 = c & 3;
        wy_reduce(acc, smem + OFF_VS, smem + OFF_SALL, tid);
        wy_apply_t<true>(smem + OFF_T, smem + OFF_SALL, tid);
        float wb[16];                                 // B operand: W[ks + 16 hh][c]
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) wb[ks] = smem[OFF_SALL + (16 * hh + ks) * 32 + c];
        // The update's A operand is the V rows this wave already holds in pa (lane c, half
        // hh: row of x[i], column c); a per-wave LDS tile (32 rows of pitch 36) turns them
        // into the rows of 16 consecutive V columns each lane needs.
        float* tile = smem + OFF_VS + wv * 32 * 36;
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
            const int ra = 2 * wv + hq + NSLOT * (16 * vb + 4 * q + e4);
            const uint32_t am = ra < h ? 0xffffffffu : 0u;
#pragma unroll
            for (int il = 0; il < 16; ++il)
                if (16 * vb + il < NR) tile[(2 * il + hh) * 36 + c] = pa[(16 * vb + il) % NR];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float va[16];
            const float* trow_p = tile + (2 * (4 * q + e4) + hq) * 36 + 16 * hh;
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                const floatx4 v4 = *reinterpret_cast<const floatx4*>(trow_p + 4 * t4);
                va[4 * t4] = v4[0]; va[4 * t4 + 1] = v4[1]; va[4 * t4 + 2] = v4[2]; va[4 * t4 + 3] = v4[3];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            floatx16 o;
#pragma unroll
            for (int r = 0; r < 16; ++r) o[r] = (16 * vb + r < NR) ? x[(16 * vb + r) % NR] : 0.f;
#pragma unroll
            for (int ks = 0; ks < 16; ++ks)
                o = __builtin_amdgcn_mfma_f32_32x32x2f32(masked(-va[ks], am), wb[ks], o, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (16 * vb + r < NR) x[16 * vb + r] = o[r];
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
    if constexpr (NR >= kTwoColMinNR) {
        panel_two_cols<NR, MODE>(d, ex, smem, x);
        return;
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
    float* colbuf = smem + OFF_COL + slot * COL_PITCH;
    for (int j = 0; j < nb; ++j) {
        const int buf = j & 1;
        const int jn = j + 1;
        // every lane sums its own column's partials; the pivot column's sum and diagonal
        // entry come from lane j of the wave (half of the LDS reads after the barrier)
        const float dc = read_d(smem, buf, c);
        const float ajc = read_row(smem, buf, c);
        const float dj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dc), j));
        const float alpha = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ajc), j));
        const Refl R = reflector(alpha, dj);
        const float sv = (c < nb && c != j) ? R.sc * (dc - R.beta * ajc) : 0.f;
        if (slot == 0) {
            smem[OFF_SALL + c * 33 + j] = sv;
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
    float* Vt = d.V + (int64_t)d.zrows * d.vld;
    if constexpr (MODE == 0) {
        // explicit V to global and to LDS (rows padded to 32 with zeros), then Y = V T
        float* Vs = smem + OFF_VS;
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
    } else {
        // explicit V and T to global; the other waves write their V rows while wave 0
        // builds the diagonal blocks of T
        auto write_v = [&]() {
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const int r = slot + NSLOT * i;
                if (r < h) {
                    float v = 0.f;
                    if (c < nb) v = (r > c) ? x[i] : (r == c ? 1.f : 0.f);
                    stg(Vt + (int64_t)r * d.vld + c, v);
                }
            }
        };
        if (wv != 0) write_v();
        build_T_diag(smem, nb, tid);
        if (wv == 0) write_v();
        __syncthreads();
        build_T_offdiag(smem, nb, tid);
        __syncthreads();
        for (int e = tid; e < PW * PW; e += PANEL_THREADS) stg(ex.T + e, smem[OFF_T + (e >> 5) * 33 + (e & 31)]);
    }
}

template <int NR>
__global__ __launch_bounds__(PANEL_THREADS) void panel_reg_kernel(const PanelDesc* __restrict__ descs) {
    extern __shared__ float smem[];
    const PanelDesc d = descs[blockIdx.x];
    const PanelExtra ex{nullptr, nullptr, nullptr, 0};
    panel_body<NR, 0>(d, ex, smem);
}

// One launch of the fused QR step.  Blocks [0, npanel) factor panels (after applying the
// previous panel's reflectors to their columns in registers); the rest apply the previous
// panel's reflectors to 32 trailing columns of P or 32 rows of Q.  The two kinds touch
// disjoint data: a panel's own columns are excluded from the trailing slabs.
template <int NR>
__global__ __launch_bounds__(PANEL_THREADS) void qr_step_kernel(const StepPanelDesc* __restrict__ panels, int npanel,
                                                                const SlabDesc* __restrict__ slabs) {
    extern __shared__ float smem[];
    const int tid = threadIdx.x;
    if ((int)blockIdx.x < npanel) {
        const StepPanelDesc sp = panels[blockIdx.x];
        const PanelExtra ex{sp.Vp, sp.Tp, sp.T, sp.nbp};
        if (sp.nbp > 0)
            panel_body<NR, 2>(sp.pd, ex, smem);
        else
            panel_body<NR, 1>(sp.pd, ex, smem);
        return;
    }
    const SlabDesc s = slabs[blockIdx.x - npanel];
    load_T(s.T, smem + OFF_T, tid);
    if (s.role == 0) {
        wy_left_product(s.V, s.vld, s.M, s.ld, s.h, s.count, smem + OFF_VS, smem + OFF_SALL, tid);
        wy_apply_t<true>(smem + OFF_T, smem + OFF_SALL, tid);
        wy_update_rows(s.V, s.vld, s.M, s.ld, s.h, s.count, smem + OFF_SALL, tid);
    } else {
        const bool ident = s.ident != 0;
        wy_right_product(s.M, s.ld, s.count, s.V, s.vld, s.h, smem + OFF_VS, smem + OFF_SALL, tid, ident, s.diag);
        wy_apply_t<false>(smem + OFF_T, smem + OFF_SALL, tid);
        wy_update_cols(s.M, s.ld, s.count, s.V, s.vld, s.h, smem + OFF_SALL, tid, ident, s.diag);
    }
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
    // Rows are visited GU at a time with every load of a batch issued before any use:
    // the panel lives in L2, and a row-at-a-time loop waits one L2 round trip per row.
    // Addresses are clamped into the panel and out-of-range values masked.
    constexpr int GU = 16;
    const int cc = c < nb ? c : nb - 1;
    {
        float pacc = 0.f, rj = 0.f;
        for (int rb = slot; rb < h; rb += NSLOT * GU) {
            float xv[GU], x0[GU];
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int r = min(rb + NSLOT * u, h - 1);
                xv[u] = Ap[(int64_t)r * ld + cc];
                x0[u] = Ap[(int64_t)r * ld];
            }
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int r = rb + NSLOT * u;
                const float x = (c < nb && r < h) ? xv[u] : 0.f;
                pacc = fmaf(x0[u], x, pacc);
                if (r == 0) rj = x;
            }
        }
        write_partial(smem, 0, c, lane, wv, pacc);
        if (slot == 0) smem[OFF_ROWJ + c] = rj;
    }
    __syncthreads();

    for (int j = 0; j < nb; ++j) {
        const int buf = j & 1;
        // every lane sums its own column's partials; the pivot column's sum and diagonal
        // entry come from lane j of the wave (half of the LDS reads after the barrier)
        const float dc = read_d(smem, buf, c);
        const float ajc = read_row(smem, buf, c);
        const float dj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dc), j));
        const float alpha = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ajc), j));
        const Refl R = reflector(alpha, dj);
        const float sv = (c < nb && c != j) ? R.sc * (dc - R.beta * ajc) : 0.f;
        if (slot == 0) {
            smem[OFF_SALL + c * 33 + j] = sv;
            if (c == 0) {
                smem[OFF_TAU + j] = R.tau;
                smem[OFF_RD + j] = R.beta;   // no global store inside the loop
            }
        }
        const float f = R.tau * sv;
        const int jn = j + 1;
        float pacc = 0.f, rj = 0.f;
        const int r0 = j + ((slot - (j & (NSLOT - 1)) + NSLOT) & (NSLOT - 1));
        // two batches in flight: the loads of batch b + 1 are issued before batch b is
        // updated (rows clamped into the panel, so every load is unconditional; rows past
        // the panel are masked where they are used)
        auto load_batch = [&](float (&xv)[GU], float (&xj)[GU], int rb) {
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int r = min(rb + NSLOT * u, h - 1);
                xv[u] = Ap[(int64_t)r * ld + cc];
                xj[u] = Ap[(int64_t)r * ld + j];
            }
        };
        auto use_batch = [&](const float (&xv)[GU], const float (&xj)[GU], int rb) {
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int r = rb + NSLOT * u;
                const bool in = r < h;
                float x = c < nb ? xv[u] : 0.f;
                const float vr = (r == j) ? 1.f : R.sc * xj[u];
                if (in && c == j) {
                    x = (r == j) ? R.beta : vr;
                    Ap[(int64_t)r * ld + c] = x;
                } else if (in && c > j && c < nb) {
                    x -= f * vr;
                    Ap[(int64_t)r * ld + c] = x;
                }
                const float xn = __shfl(x, jn, 32);
                if (in && r >= jn) pacc += xn * x;
                if (in && r == jn) rj = x;
            }
        };
        {
            float xa[GU], ja[GU], xb[GU], jb[GU];
            load_batch(xa, ja, r0);
            for (int rb = r0; rb < h; rb += 2 * NSLOT * GU) {
                load_batch(xb, jb, rb + NSLOT * GU);
                use_batch(xa, ja, rb);
                load_batch(xa, ja, rb + 2 * NSLOT * GU);
                use_batch(xb, jb, rb + NSLOT * GU);
            }
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

template <int NR>
hipError_t launch_step(const StepPanelDesc* panels, int npanel, const SlabDesc* slabs, int nslab, int max_h,
                       hipStream_t stream) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&qr_step_kernel<NR>), hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)qr_step_lds_bytes(NSLOT * NR < PANEL_LDS_MAX_ROWS ? NSLOT * NR : PANEL_LDS_MAX_ROWS));
    if (attr != hipSuccess) return attr;
    S4_LAUNCH(qr_step_kernel<NR>, dim3(npanel + nslab), dim3(PANEL_THREADS), qr_step_lds_bytes(max_h), stream,
              panels, npanel, slabs);
    return hipGetLastError();
}

}  // namespace

// rows of the layout hand-over buffer of a panel of up to max_h rows (two-column path)
static int handover_rows(int max_h) {
    const int nr = panel_rows_class(max_h < 1 ? 1 : max_h);
    return nr >= kTwoColMinNR ? NSLOT * nr : 0;
}

size_t qr_step_lds_bytes(int max_h) {
    // the fused panel keeps V in registers and writes it to global directly; LDS holds the
    // fixed panel area and the partial products of the block applications or the layout
    // hand-over of a tall panel
    const int tail = handover_rows(max_h) * 33 > WY_PART ? handover_rows(max_h) * 33 : WY_PART;
    return (size_t)(OFF_VS + tail) * sizeof(float);
}

hipError_t launch_qr_step(int rows_class, const StepPanelDesc* panels, int npanel, const SlabDesc* slabs,
                          int nslab, int max_h, hipStream_t stream) {
    if (npanel + nslab <= 0) return hipSuccess;
    switch (rows_class) {
#define S4_CASE(N) case N: return launch_step<N>(panels, npanel, slabs, nslab, max_h, stream);
        S4_PANEL_CLASSES(S4_CASE)
#undef S4_CASE
        default: return hipErrorInvalidValue;
    }
}

int panel_rows_class(int h) {
    if (h > PANEL_LDS_MAX_ROWS) return 0;
    for (int i = 0; i < PANEL_NCLASS; ++i)
        if (NSLOT * PANEL_CLASSES[i] >= h) return PANEL_CLASSES[i];
    return 0;
}

size_t panel_lds_bytes(bool in_regs, int max_h) {
    const size_t fixed = (size_t)OFF_VS * sizeof(float);
    const int hpad = (max_h + 31) & ~31;
    const int rows = handover_rows(max_h) > hpad ? handover_rows(max_h) : hpad;
    return fixed + (in_regs ? (size_t)rows * 33 * sizeof(float) : 0);
}

hipError_t launch_panel(int rows_class, const PanelDesc* descs, int ndesc, int max_h,
                        hipStream_t stream) {
    if (ndesc <= 0) return hipSuccess;
    switch (rows_class) {
#define S4_CASE(N) case N: return launch_reg<N>(descs, ndesc, max_h, stream);
        S4_PANEL_CLASSES(S4_CASE)
#undef S4_CASE
        default: break;
    }
    const size_t lds = panel_lds_bytes(false, max_h);
    S4_LAUNCH(panel_global_kernel, dim3(ndesc), dim3(PANEL_THREADS), lds, stream, descs);
    return hipGetLastError();
}

}  // namespace s4
