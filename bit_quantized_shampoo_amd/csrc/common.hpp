// Shared device-side types for the 4-bit Shampoo kernels (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s4 {

// Optional start/stop events for the next kernel launch.  A timed launch goes through
// hipExtLaunchKernelGGL, which records the events in the dispatch itself, so it measures
// the kernel alone (no separate event packets); untimed launches (and launches under
// graph capture) are plain hipLaunchKernelGGL.
struct LaunchTiming {
    hipEvent_t start = nullptr, stop = nullptr;
};
inline LaunchTiming& launch_timing() {
    static thread_local LaunchTiming t;
    return t;
}
#define S4_LAUNCH(kernel, grid, block, shmem, stream, ...)                                         \
    do {                                                                                          \
        ::s4::LaunchTiming& lt_ = ::s4::launch_timing();                                          \
        if (lt_.start)                                                                            \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, lt_.start, lt_.stop, 0, __VA_ARGS__); \
        else                                                                                      \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                  \
        lt_.start = lt_.stop = nullptr;                                                           \
    } while (0)

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Loads and stores through the global address space.  Pointers taken from descriptor
// tables are generic (flat) to the compiler; flat accesses also count against the LDS
// wait counter, so every LDS wait of a kernel would also wait for its in-flight global
// prefetches.  Casting to address space 1 emits global_load / global_store instead.
template <class T>
__device__ __forceinline__ T ldg(const T* p) {
    using G = __attribute__((address_space(1))) const T;
    return *(G*)p;
}
template <class T>
__device__ __forceinline__ void stg(T* p, T v) {
    using G = __attribute__((address_space(1))) T;
    *(G*)p = v;
}
// Streaming forms for data touched once (the codec's fp32 side): the nontemporal hint
// keeps single-use lines from displacing reused ones and lets the memory system stream them.
template <class T>
__device__ __forceinline__ T ldg_nt(const T* p) {
    using G = __attribute__((address_space(1))) const T;
    return __builtin_nontemporal_load((G*)p);
}
template <class T>
__device__ __forceinline__ void stg_nt(T* p, T v) {
    using G = __attribute__((address_space(1))) T;
    __builtin_nontemporal_store(v, (G*)p);
}

// Per-block user pointers of one call, uploaded once per call; descriptors refer
// to an entry by index so that the static descriptor tables never change.
struct IoEntry {
    const float* G;
    int64_t ldg;
    float* P;
    int64_t ldp;
};

// One matrix product D = alpha * op(A) op(B) [* rscale rows][* cscale cols] + beta * C.
// op(B)'s row k is multiplied by kscale[k] when kscale is set.  A pointer given by an
// io index (>= 0) is taken from the call's io table instead of the field.
// Split K: with ksplit > 1 the K range is cut into chunks of kchunk and chunk s writes
// its partial product (beta must be 0) to D + s * dslab.  A consumer reads such
// partials back summed: op(A) = sum_{s < anslab} A[s * aslab ...] (same for B).
// Most split-K partial slabs a GEMM operand may sum while loading.
constexpr int GEMM_MAX_SLABS = 8;

struct GemmDesc {
    const float* A;
    const float* B;
    const float* C;
    float* D;
    const float* kscale;
    const float* rscale;
    const float* cscale;
    int64_t lda, ldb, ldc, ldd;
    int64_t aslab, bslab, dslab;
    int32_t M, N, K;
    int32_t tiles_m;          // tiles along M for the launch's tile shape
    float alpha, beta;
    int32_t a_io, b_io, d_io; // -1 or index into the io table (A/B = G, D = P)
    int32_t flags;            // GEMM_F_* below
    int32_t ksplit, kchunk, anslab, bnslab;
    int32_t pad0, pad1;
};
static_assert(sizeof(GemmDesc) == 176, "GemmDesc layout");
enum : int32_t {
    GEMM_F_TA = 1,            // op(A) = A^T
    GEMM_F_TB = 2,            // op(B) = B^T
    GEMM_F_COLDOT = 4,        // epilogue: D[tile_m][col] = sum over the tile's rows of
                              //   alpha * (op(A) op(B))[row][col] * C[row][col]; ldd = row stride
    GEMM_F_SYM = 8,           // the result is symmetric (M == N, square tiles, no row or column
                              //   scale, C symmetric): only tiles on or above the diagonal are
                              //   computed; an off-diagonal tile is also stored transposed
};

// Codec work item: one flattened matrix of n fp32 elements.
struct CodecDesc {
    const uint8_t* codes_in;  // dequant source
    const float* scales_in;
    uint8_t* codes_out;       // quant destination
    float* scales_out;
    const float* x_in;        // quant source
    float* x_out;             // dequant destination
    int64_t n;
    int64_t pad;
};
static_assert(sizeof(CodecDesc) == 64, "CodecDesc layout");

// One Householder panel of one matrix: rows c0.., columns c0..c0+nb-1 of A.
struct PanelDesc {
    float* A;                 // matrix base (p x p)
    float* V;                 // out: explicit unit-lower reflector vectors, 32 columns
    float* Y;                 // out: V T (compact WY), same shape and pitch as V
    float* rdiag;             // out: R diagonal, entries c0..c0+nb-1
    int64_t ld;               // of A
    int64_t vld;              // row pitch of V and Y
    int32_t c0, h, nb;
    int32_t zrows;            // V and Y start zrows rows above the panel's top row; those
                              // rows are written as zeros
};
static_assert(sizeof(PanelDesc) == 64, "PanelDesc layout");

// One panel of a fused QR step: the panel, and the reflector block of the panel before it,
// which the workgroup first applies to this panel's columns (nbp == 0: none).  The panel
// writes V (pd.V) and its 32 x 32 T (row-major) instead of Y.
struct StepPanelDesc {
    PanelDesc pd;
    const float* Vp;          // previous panel's V, top row pd.c0 - nbp, pitch pd.vld
    const float* Tp;          // previous panel's T
    float* T;                 // this panel's T
    int32_t hp, nbp;          // rows of Vp (pd.h + nbp) and its reflector count
};
static_assert(sizeof(StepPanelDesc) == 96, "StepPanelDesc layout");

// One slab of a fused QR step: a reflector block (V: h rows, 32 columns of which the first
// nb are reflectors, pitch vld; T: 32 x 32) applied as M <- M - V (T^T (V^T M)) to
// `count` <= 32 columns of P (role 0; M points at row r0 of the first column, h rows) or as
// M <- M - ((M V) T) V^T to `count` <= 32 rows of Q (role 1; M points at column r0 of the
// first row, h columns).
// Role 1 with ident = 1: M holds the identity on input (Q's first block application):
// M[m][k] is read as 1 where m + diag == k, else 0, and M's memory is only written.
struct SlabDesc {
    float* M;
    const float* V;
    const float* T;
    int64_t ld;               // of M
    int64_t vld;
    int32_t role, h;
    int32_t count, ident;
    int64_t diag;
};
static_assert(sizeof(SlabDesc) == 64, "SlabDesc layout");

// One block of the grafting epilogue: rows of G, P (io table entry `blk`) and of W, M, V
// (graft io table entry `blk`) in tiles of `rows` rows; `parts` receives two partial
// sums per tile (||d_graft||^2 and ||P||^2 over the tile).
struct GraftDesc {
    float* parts;
    int32_t m, n, rows, blk;
    int32_t ntiles, pad0;
};
static_assert(sizeof(GraftDesc) == 32, "GraftDesc layout");

// One matrix of the coupled Newton inverse root: the caller's input and output (with
// their leading dimensions), the contiguous p x p source and destination of an
// elementwise step, the identity target of the initial step, the per-row-tile partial
// sums of the Frobenius norm and the matrix's scale slot.
struct NewtonDesc {
    const float* A;
    float* out;
    const float* src;
    float* dst;
    float* ident;
    float* parts;
    float* scale;
    int64_t lda, ldo;
    int32_t p, pad;
};
static_assert(sizeof(NewtonDesc) == 80, "NewtonDesc layout");

// Per-call entry of the graft io table (same layout as shampoo4_graft_io).
struct GraftIo {
    float* W;
    int64_t ldw;
    float* M;
    float* V;
};

// Column / vector work item for the small elementwise kernels.
struct VecDesc {
    const float* a;           // e.g. Q
    const float* b;           // e.g. L~ Q
    float* out;               // e.g. eigenvalues / root scaling / W
    const float* aux;         // e.g. R diagonal
    uint8_t* codes;           // identity init
    float* scales;
    int64_t ld;
    int32_t p, rows;          // rows: number of partial rows (Rayleigh reduction)
};
static_assert(sizeof(VecDesc) == 64, "VecDesc layout");

// Initial state of one side: U = I (codes and scales), lam = 0, root = (I, d = 1).
enum : int32_t {
    INIT_4BIT = 0,            // U as 4-bit codes and scales
    INIT_FP32 = 1,            // U kept in float32: codes/rcodes hold p x p floats, no scales
    INIT_DIAG = 2,            // diagonal side: only lam = 0 and d = 1
};
struct InitDesc {
    uint8_t* codes;
    float* scales;
    float* lam;
    uint8_t* rcodes;
    float* rscales;
    float* d;
    int32_t p;
    int32_t kind;             // INIT_*
};
static_assert(sizeof(InitDesc) == 56, "InitDesc layout");

// One block with a diagonal side (the fallback for a side over the size threshold):
// G (and P) through io entry `blk`; rowpart [tiles_n][m] receives partial row sums of G^2
// (side L diagonal), colpart [tiles_m][n] partial column sums (side R diagonal); d_l and
// d_r are the root scalings of a block whose two sides are diagonal (P = diag(d_l) G
// diag(d_r)).
struct DiagDesc {
    float* rowpart;
    float* colpart;
    const float* d_l;
    const float* d_r;
    int32_t m, n, blk, tiles_n;
};
static_assert(sizeof(DiagDesc) == 48, "DiagDesc layout");

// One float64 product of the float64 statistics update: D = alpha op(A) op(B) + beta C,
// op(B)'s row k times kscale[k] when set.  A and B are double, or float for a launch
// whose operands are the caller's gradients (a_io / b_io: taken from the io table).
struct Gemm64Desc {
    const void* A;
    const void* B;
    const double* C;
    double* D;
    const float* kscale;
    int64_t lda, ldb, ldc, ldd;
    double alpha, beta;
    int32_t M, N, K, tiles_m;
    int32_t a_io, b_io;
};
static_assert(sizeof(Gemm64Desc) == 112, "Gemm64Desc layout");

// One float64 Householder panel: rows c0.., columns c0..c0+nb-1 (nb <= 32) of the p x p
// matrix A (leading dimension ld); V and Y = V T receive h x 32 (pitch vld; columns past
// nb zero), rdiag[c0 + j] the diagonal of R.
struct Panel64Desc {
    double* A;
    double* V;
    double* Y;
    double* rdiag;
    int64_t ld, vld;
    int32_t c0, h, nb, pad;
};
static_assert(sizeof(Panel64Desc) == 64, "Panel64Desc layout");

// Float64 per-column / conversion work item on a p x p matrix (leading dimension p).
struct Vec64Desc {
    const double* a;          // coldot: Q; ident: R diagonal; cvt (to float32): source
    const double* b;          // coldot: W = L~ Q
    double* out;              // ident: Q; cvt (to float64): destination
    float* f32;               // coldot: eigenvalues; cvt: the float32 side
    int32_t p, pad;
};
static_assert(sizeof(Vec64Desc) == 40, "Vec64Desc layout");

// Find the work item owning `tile` from an inclusive-exclusive prefix of tile counts.
__device__ __forceinline__ int find_item(const int* __restrict__ prefix, int n, int tile) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace s4
