// Host-side launchers of the gfx950 kernels.  Every launcher enqueues one kernel on
// `stream` and returns the launch status; work items are described by device
// descriptor arrays plus an exclusive prefix of per-item tile counts.
#pragma once

#include "common.hpp"
#include "shampoo4.h"

namespace s4 {

// Tile shapes of the fp32 MFMA GEMM (workgroup of 4 waves).
// tile shapes (the first GEMM_NCFG are the shape classes); GEMM_64x64_K2: the 64 x 64
// tile with two groups of four waves splitting K (16-byte loads, no split-K slabs)
// GEMM_X3 / GEMM_X3_64: the bf16 matrix cores with each fp32 operand split into three
// bf16 pieces (gemm_x3.hip; tile GEMM_X3_BM x GEMM_X3_BN, or 64 x 64), for launches that
// would take 128 x 128 (64 x 64) tiles and sum no split-K slabs.
enum GemmCfg { GEMM_128x128 = 0, GEMM_64x64 = 1, GEMM_32x128 = 2, GEMM_128x32 = 3, GEMM_NCFG = 4,
               GEMM_64x64_K2 = 5, GEMM_X3 = 6, GEMM_X3_64 = 7 };
inline bool gemm_cfg_x3(int cfg) { return cfg == GEMM_X3 || cfg == GEMM_X3_64; }
constexpr int GEMM_MODE_MIXED = -1;   // descriptors of one launch carry different transposes
void gemm_tile_dims(int cfg, int* bm, int* bn);
// mode: GEMM_F_TA | GEMM_F_TB shared by all descriptors, or GEMM_MODE_MIXED.
// vec: every operand of every descriptor has a 16-byte aligned base (after io
// indirection), a pitch and a contiguous extent that are multiples of 4, and slab
// strides that are multiples of 4 (gemm_vec_ok on the host).
// slab: some descriptor sums split-K slabs while loading (anslab or bnslab > 1).
// kscale: some descriptor scales op(B)'s rows (selects the kernels that load the scale).
hipError_t launch_gemm(int cfg, int mode, bool vec, bool slab, bool kscale, const GemmDesc* descs,
                       const int* prefix, int ndesc, int ntiles, const IoEntry* io, hipStream_t stream);
// The three-piece bf16 product (no split-K slab sums; vec as for launch_gemm, with every
// operand under 2 GiB) on 128 x 128 tiles (2 x 2 waves of 2 x 2 blocks of 32 x 32).
constexpr int GEMM_X3_BM = 128, GEMM_X3_BN = 128;
hipError_t launch_gemm_x3(bool small, int mode, bool vec, bool kscale, const GemmDesc* descs, const int* prefix,
                          int ndesc, int ntiles, const IoEntry* io, hipStream_t stream);
// The allocation-free batched GEMM keeps its descriptor table and tile prefix (one 256-byte
// aligned piece each) in a static device array of this size per GPU.
constexpr size_t GEMM_STATIC_SCRATCH_BYTES = 384 * 1024;
// The device address of the current device's array (looked up on its first use).
hipError_t gemm_static_scratch(void** out);
// Host check of the 16-byte-load conditions of one descriptor, operands given through
// the io table excepted (their pointers and pitches are checked per call).
bool gemm_vec_ok(const GemmDesc& d);

// Codec: elements per workgroup tile.
constexpr int DEQ_TILE = 4096;     // 256 threads x 4 quads x 4 elements
constexpr int QUANT_TILE = 4096;   // 256 threads x 4 quads x 4 elements
constexpr int COPY_TILE = 8192;    // bytes of codes per workgroup
// workgroups for n elements (quantization blocks of 64 padded)
inline int64_t dequant_tiles(int64_t n) { return ((n + 63) / 64 * 64 + DEQ_TILE - 1) / DEQ_TILE; }
inline int64_t quant_tiles(int64_t n) { return ((n + 63) / 64 * 64 + QUANT_TILE - 1) / QUANT_TILE; }
// codebook: SHAMPOO4_CODEBOOK_LINEAR_SQUARE or SHAMPOO4_CODEBOOK_DYNAMIC_TREE
hipError_t launch_dequant(int codebook, const CodecDesc* descs, const int* prefix, int ndesc, int ntiles,
                          hipStream_t stream);
hipError_t launch_quant(int codebook, const CodecDesc* descs, const int* prefix, int ndesc, int ntiles,
                        uint32_t* flag, hipStream_t stream);
hipError_t launch_dequant_single(int codebook, const CodecDesc& d, hipStream_t stream);
hipError_t launch_quant_single(int codebook, const CodecDesc& d, hipStream_t stream);
hipError_t launch_codec_copy(const CodecDesc* descs, const int* prefix, int ndesc, int ntiles,
                             hipStream_t stream);
bool host_codebook(int codebook, float levels[16], float midpoints[15]);

// Householder panel factorization, one workgroup per panel.  Panels of height
// h <= 16 * rows_class (rows_class from PANEL_CLASSES: rows per lane) keep the panel in
// registers; rows_class 0 works on taller panels in place in global memory.
constexpr int PANEL_THREADS = 512;
constexpr int PANEL_LDS_MAX_ROWS = 1024;
constexpr int PANEL_NCLASS = 12;
constexpr int PANEL_CLASSES[PANEL_NCLASS] = {2, 4, 8, 12, 16, 20, 24, 32, 40, 48, 56, 64};
#define S4_PANEL_CLASSES(X) X(2) X(4) X(8) X(12) X(16) X(20) X(24) X(32) X(40) X(48) X(56) X(64)
int panel_rows_class(int h);
size_t panel_lds_bytes(bool in_regs, int max_h);
// Fused QR step: npanel panel workgroups (each first applying the previous panel's
// reflectors to its own columns, then factoring them) and nslab slab workgroups (the
// previous panel's reflectors on trailing columns of P and on rows of Q) in one launch.
// rows_class: register class of the tallest panel (2 when npanel == 0).
size_t qr_step_lds_bytes(int max_h);
hipError_t launch_qr_step(int rows_class, const StepPanelDesc* panels, int npanel, const SlabDesc* slabs,
                          int nslab, int max_h, hipStream_t stream);
hipError_t launch_panel(int rows_class, const PanelDesc* descs, int ndesc, int max_h,
                        hipStream_t stream);

// Small per-column / per-element kernels.
constexpr int FILL_TILE = 4096;              // elements per workgroup (at least one row)
constexpr int fill_rows(int p) { return p >= FILL_TILE ? 1 : FILL_TILE / p; }
constexpr int fill_tiles(int p) { return (p + fill_rows(p) - 1) / fill_rows(p); }
// lam_j = max(sum_t partial[t][j], 0) over the per-tile partial rows of the fused
// column-dot GEMM epilogue
hipError_t launch_rayleigh_reduce(const VecDesc* descs, const int* prefix, int ndesc, int ntiles,
                                  uint32_t* flag, hipStream_t stream);
// with_signs: diag(sign(aux)) (0 -> +) instead of I
hipError_t launch_identity_fill(const VecDesc* descs, const int* prefix, int ndesc, int ntiles, bool with_signs,
                                hipStream_t stream);
hipError_t launch_sign_flip(const VecDesc* descs, const int* prefix, int ndesc, int ntiles,
                            hipStream_t stream);
hipError_t launch_root_scaling(const VecDesc* descs, const int* prefix, int ndesc, int ntiles,
                               float eps, uint32_t* flag, hipStream_t stream);
hipError_t launch_identity_state(const InitDesc* descs, const int* prefix, int ndesc, int ntiles,
                                 hipStream_t stream);
// out[0..n) = a[0..n) (n = desc.ld), 16-byte vectors; with a flag, non-finite values raise it
constexpr int COPYF_TILE = 4096;             // elements per workgroup
hipError_t launch_copyf(const VecDesc* descs, const int* prefix, int ndesc, int ntiles, uint32_t* flag,
                        hipStream_t stream);

// Coupled Newton inverse 4th root: elementwise steps (row tiles of fill_rows(p) rows).
hipError_t launch_newton_norm(const NewtonDesc* descs, const int* prefix, int ndesc, int ntiles, float eps,
                              hipStream_t stream);
hipError_t launch_newton_scale(const NewtonDesc* descs, int ndesc, hipStream_t stream);
// mode 0: scaled damped input and identity; 1: F = 1.25 I - 0.25 M; 2: scaled result out
hipError_t launch_newton_elem(const NewtonDesc* descs, const int* prefix, int ndesc, int ntiles, int mode,
                              float eps, hipStream_t stream);

// Diagonal fallback: partial sums of G^2 over tiles of DIAG_TR rows x DIAG_TC columns,
// their EMA into the diagonal statistic, and P = diag(d_L) G diag(d_R).
constexpr int DIAG_TR = 32;
constexpr int DIAG_TC = 256;
constexpr int diag_scale_rows(int n) { return n >= 4096 ? 1 : 4096 / n; }
hipError_t launch_diag_partials(const DiagDesc* descs, const int* prefix, int ndesc, int ntiles,
                                const IoEntry* io, hipStream_t stream);
// out_j = beta out_j + (1 - beta) sum_{t < rows} a[t * ld + j] (VecDesc: a, out, ld, p, rows)
hipError_t launch_diag_ema(const VecDesc* descs, const int* prefix, int ndesc, int ntiles, float beta,
                           uint32_t* flag, hipStream_t stream);
hipError_t launch_diag_scale(const DiagDesc* descs, const int* prefix, int ndesc, int ntiles,
                             const IoEntry* io, hipStream_t stream);

// Float64 statistics update: the matrix product on the fp64 matrix cores (128 x 128 tiles;
// mode GEMM_F_TA | GEMM_F_TB shared by the launch; in_float: the operands are float,
// else double), Householder panels, Rayleigh quotients, the signed identity start of Q
// and the float32 <-> float64 conversions (CVT_TILE elements per workgroup).
int gemm64_tiles(int M, int N);
int gemm64_tiles_m(int M);
hipError_t launch_gemm64(int mode, bool in_float, const Gemm64Desc* descs, const int* prefix, int ndesc,
                         int ntiles, const IoEntry* io, hipStream_t stream);
hipError_t launch_panel64(const Panel64Desc* descs, int ndesc, hipStream_t stream);
hipError_t launch_coldot64(const Vec64Desc* descs, const int* prefix, int ndesc, int ntiles, uint32_t* flag,
                           hipStream_t stream);
hipError_t launch_ident64(const Vec64Desc* descs, const int* prefix, int ndesc, int ntiles, hipStream_t stream);
constexpr int CVT_TILE = 4096;
hipError_t launch_cvt(const Vec64Desc* descs, const int* prefix, int ndesc, int ntiles, int dir,
                      hipStream_t stream);

// Grafting epilogue: two launches over the same row tiles of every block.
constexpr int GRAFT_TILE = 4096;             // elements per workgroup (at least one row)
constexpr int graft_rows(int n) { return n >= GRAFT_TILE ? 1 : GRAFT_TILE / n; }
struct GraftParams {
    int mode;                                // 0 SGD, 1 Adam
    float lr, eps_graft, beta1, beta2, eps_adam;
    float c1, c2;                            // Adam bias corrections 1 - beta^t
};
hipError_t launch_graft_norms(const GraftDesc* descs, const int* prefix, int ndesc, int ntiles,
                              const IoEntry* io, const GraftIo* gio, GraftParams prm, uint32_t* flag,
                              hipStream_t stream);
hipError_t launch_graft_apply(const GraftDesc* descs, const int* prefix, int ndesc, int ntiles,
                              const IoEntry* io, const GraftIo* gio, GraftParams prm, hipStream_t stream);

}  // namespace s4
