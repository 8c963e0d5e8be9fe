/*
 * shampoo4.h -- C ABI of the 4-bit Shampoo preconditioner step for MI355X (gfx950).
 *
 * The method ("4-bit Shampoo for Memory-Efficient Network Training", abstract;
 * "Shampoo -- Second-Order Optimizer", sections "Kronecker factorization",
 * "Where the fourth root comes from", "Rotation, not just rescaling",
 * "Computing the inverse fourth root", "The cost dial", "Pitfalls"):
 * for every weight block G:[m,n] two Kronecker factors L:[m,m] and R:[n,n] are
 * kept, each as a 4-bit eigenvector matrix U (block-wise linear-square codes,
 * one fp32 absmax scale per 64 consecutive elements of U flattened row-major,
 * eigenvectors in the columns) plus fp32 eigenvalues.  A step
 *
 *   update_stats(G):  V = Bjorck^k(dequant(U))  (V <- 1.5 V - 0.5 V V^T V)
 *                     L~ = beta V diag(lam) V^T + (1 - beta) G G^T
 *                     Q R = L~ V (Householder, diag R >= 0)
 *                     lam_i = max(q_i^T L~ q_i, 0),  U <- quant(Q)
 *                     (side R: G^T in place of G)
 *   refresh_root():   d_i = (lam_i + eps)^(-1/4), root codes <- codes
 *   precondition(G):  V^r = Bjorck^k(dequant(root codes)) per side,
 *                     P = V^r_L diag(d_L) V^r_L^T G V^r_R diag(d_R) V^r_R^T
 *
 * Conventions shared by every entry point:
 *  - All matrices are fp32, row-major, with an explicit leading dimension
 *    (elements, >= number of columns).  G and P of a block may be strided
 *    views into a larger weight matrix.
 *  - Pointers named "device" are HIP device pointers; everything else is
 *    host memory.  The caller owns all device memory (state and workspace
 *    buffers, G, P): the library never allocates or frees device memory.
 *    The only memory the library allocates is host memory inside the context
 *    (descriptor tables and a small pinned staging ring), freed by
 *    shampoo4_destroy.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously on it; unless stated otherwise a call
 *    returns without waiting for the device.  Calls on one context must be
 *    ordered on one stream (or externally synchronized): they share the
 *    context's workspace.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    failed validation returns an error and enqueues nothing.
 *  - A context is not thread-safe; separate contexts are independent.
 */
#ifndef SHAMPOO4_H
#define SHAMPOO4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SHAMPOO4_ABI_VERSION 1

#if defined(__GNUC__) || defined(__clang__)
#define SHAMPOO4_API __attribute__((visibility("default")))
#else
#define SHAMPOO4_API
#endif

typedef struct shampoo4_ctx_s* shampoo4_ctx;

typedef enum {
    SHAMPOO4_OK = 0,
    SHAMPOO4_EINVAL = 1,      /* null pointer, bad config value, bad index */
    SHAMPOO4_ESHAPE = 2,      /* a block dimension outside [1, 8192] (a diagonal side: [1, 65536]),
                                 or ld < cols */
    SHAMPOO4_EALIGN = 3,      /* a state/workspace buffer not 256-byte aligned */
    SHAMPOO4_ESMALLBUF = 4,   /* buffer smaller than shampoo4_plan reported */
    SHAMPOO4_EHIP = 5,        /* a HIP runtime call or kernel launch failed */
    SHAMPOO4_ENONFINITE = 6   /* device saw NaN/Inf (reported by shampoo4_check) */
} shampoo4_status;

/* Config flags. */
#define SHAMPOO4_FLAG_ROOT_CACHE 1u   /* keep the rectified fp32 root eigenvectors in the
                                         workspace between calls: refresh_root computes them
                                         once, together with the root matrices
                                         V^r diag(d) V^r^T of both sides, precondition
                                         multiplies by those (two products per block instead
                                         of four), and an update_stats that directly follows
                                         a refresh_root reuses the eigenvectors as its own
                                         rectified eigenvectors (identical values).  Without
                                         the flag precondition recomputes them. */
#define SHAMPOO4_FLAG_KEEP_STATE 2u   /* shampoo4_init: do not write the initial state;
                                         the state buffer already holds a saved state. */
/* Schedule of the Householder QR (same results either way up to rounding order).  By
   default the plan picks from the total work W = sum over sides of p^3: reflectors reach
   the trailing matrix and Q in blocks of 128 columns (256 for orders from 2048) when
   W >= 16 * 2^30 (throughput: large batches), else panel by panel (32 columns) on the
   caller's stream.  In blocks, a batch of two or more blocks of orders below 2048
   factors alternate blocks on a second stream of the context (default priority), forked
   from the caller's stream and joined back to it within the call.
   QR_BLOCKED   always blocks;
   QR_LOOKAHEAD 32-column panels; the caller's stream carries only the chain of panels
                and each panel's update of the next panel, a second stream of the context
                (default priority) the trailing and Q updates.
   Setting both is EINVAL. */
#define SHAMPOO4_FLAG_QR_BLOCKED 4u
#define SHAMPOO4_FLAG_QR_LOOKAHEAD 8u
/* The 32-bit baseline the 4-bit method is measured against ("4-bit Shampoo ..." abstract:
   performance comparable to the 32-bit counterpart): the eigenvector matrices U are kept
   in float32 (state buffers CODES / ROOT_CODES hold p x p floats, SCALES / ROOT_SCALES are
   empty) and every stage runs the same kernels with the codec replaced by copies. */
#define SHAMPOO4_FLAG_FP32_STATE 16u
/* Replay shampoo4_update_stats from a HIP graph captured at the first call (one graph
   per variant: with or without the cached rectified eigenvectors, and with or without
   16-byte loads of the gradients, which need every G 16-byte aligned with ldg a
   multiple of 4): the kernels, and the second stream of QR_LOOKAHEAD or of the blocked
   QR with its event dependencies, are submitted as one graph launch instead of one host
   call each.  The io upload stays a separate copy before the
   launch.  While kernel timing is on, and if a capture fails, calls launch eagerly. */
#define SHAMPOO4_FLAG_GRAPHS 32u
/* Code the eigenvector matrices (U and the root snapshot) with the 4-bit dynamic tree
   codebook instead of linear-square: the alternative the abstract of "4-bit Shampoo ..."
   compares linear-square with (it reports linear-square slightly ahead).  Every stage is
   unchanged but the codec's level table.  EINVAL together with FP32_STATE. */
#define SHAMPOO4_FLAG_DT_CODEBOOK 64u
/* Run the statistics update in float64 ("Shampoo -- Second-Order Optimizer", "Computing the
   inverse fourth root": do the root in float64, since float32 eigensolvers lose the small
   eigenvalues of a near-singular accumulator; "Pitfalls": root in float64, store in fp32):
   from the dequantized eigenvectors (exact in float32) on, Bjorck, the statistic, the
   power step, the Householder QR and the Rayleigh quotients are computed in float64 on the
   fp64 matrix cores, and Q is rounded to float32 for the quantizer; the stored state, the
   root and the preconditioned direction stay float32.  Eigenvalues are then resolved down
   to about p 2^-53 lam_max instead of p 2^-24 lam_max.  The QR runs panel by panel (32
   columns); EINVAL together with QR_LOOKAHEAD or FP32_STATE.  The workspace holds the float64 matrices
   instead of most float32 ones (about 84 p^2 bytes per side against 48 p^2). */
#define SHAMPOO4_FLAG_FP64_REFRESH 128u
/* Matrix products of launches on 128 x 128 and 64 x 64 tiles (the statistics GG^T / G^TG
   and V diag(lam) V^T of "Kronecker factorization", Bjorck's V^T V and V (V^T V) of the
   rectification, the power step, Householder and Rayleigh products and the
   preconditioner sandwich; not the skinny panel-width products of the blocked QR nor
   products whose operands sum split-K slabs) run by default on the bf16 matrix cores:
   every fp32 operand element is split exactly into three bf16 pieces (x = x1 + x2 + x3,
   eight significant bits each) and the six partial products of order >= 2^-16
   (x1y1, x1y2, x2y1, x1y3, x3y1, x2y2) are accumulated in fp32.  The dropped products are
   below 2^-26 |xy|, so the error bound is the fp32 matrix cores' (about K |a||b| 2^-24 per
   entry); six 32x32x16 bf16 instructions take 6/16 of the time of the fp32 instructions
   for the same work.  Results differ from the fp32 kernel's in rounding order only.
   This flag keeps every product on the fp32 matrix cores (v_mfma_f32_32x32x2_f32). */
#define SHAMPOO4_FLAG_FP32_MFMA 256u
/* Debug checks (costly; results are unchanged): shampoo4_init checks that every
   matrix-product and codec descriptor it builds stays inside the state or the workspace
   (EINVAL otherwise), and every call that enqueues work first fills the workspace
   temporaries (all but the io tables, the device flag, the rectified root eigenvectors,
   the cached root matrices and the descriptor tables) with NaN, so a kernel that reads a
   temporary before writing it in the same call yields NaN (raised by shampoo4_check).
   With SHAMPOO4_FLAG_GRAPHS the fill is enqueued outside the captured graph. */
#define SHAMPOO4_FLAG_DEBUG 512u

/* 4-bit codebooks (16 levels, ascending, code = index; the zero level is code 7).
   LINEAR_SQUARE: sign(t) t^2 on t = -1 + 2j/15 with the j = 7 level exactly 0; times 225:
     -225 -169 -121 -81 -49 -25 -9 0 1 9 25 49 81 121 169 225.
   DYNAMIC_TREE (defined by the 8-bit optimizers paper the pages cite; not on the pages):
     a sign bit and three magnitude bits whose leading zeros E are a base-10 exponent,
     then an indicator bit and 2 - E linear fraction bits, the midpoints of equal bins of
     [0.1, 1] times 10^-E; zero; and +1 in place of the negative zero, so that a block's
     maximum is exact.  Times 2000:
     -1775 -1325 -875 -425 -155 -65 -11 0 11 65 155 425 875 1325 1775 2000. */
#define SHAMPOO4_CODEBOOK_LINEAR_SQUARE 0
#define SHAMPOO4_CODEBOOK_DYNAMIC_TREE 1

typedef struct {
    int32_t m, n;             /* block shape: G is [m, n]; side L has order m, side R order n */
} shampoo4_shape;

typedef struct {
    float beta;               /* EMA factor of the statistics, in [0, 1] */
    float eps;                /* damping added to the eigenvalues before the -1/4 power, >= 0 */
    int32_t qblock;           /* elements per quantization block; only 64 is supported */
    int32_t bjorck_iters;     /* Bjorck iterations k, 0..16 */
    int32_t power_iters;      /* subspace-iteration steps per update, 1..8 */
    uint32_t flags;           /* SHAMPOO4_FLAG_* */
} shampoo4_config;

typedef struct {
    const float* G;           /* device, [m, n] gradient of the block, row-major */
    int64_t ldg;              /* leading dimension of G (elements), >= n */
    float* P;                 /* device, [m, n] output (precondition only; may be NULL for
                                 update_stats), row-major; must not overlap G */
    int64_t ldp;              /* leading dimension of P (elements), >= n */
} shampoo4_io;

/* Which buffer shampoo4_layout describes. */
typedef enum {
    SHAMPOO4_BUF_CODES = 0,       /* state: uint8 [nqb*32] packed codes of U */
    SHAMPOO4_BUF_SCALES = 1,      /* state: fp32 [nqb] block scales of U */
    SHAMPOO4_BUF_EIG = 2,         /* state: fp32 [p] eigenvalues lam */
    SHAMPOO4_BUF_ROOT_CODES = 3,  /* state: uint8 [nqb*32] root codes */
    SHAMPOO4_BUF_ROOT_SCALES = 4, /* state: fp32 [nqb] root scales */
    SHAMPOO4_BUF_ROOT_D = 5,      /* state: fp32 [p] root scaling d */
    SHAMPOO4_BUF_V = 16,          /* workspace: fp32 [p,p] rectified eigenvectors of the
                                     last update_stats */
    SHAMPOO4_BUF_STAT = 17,       /* workspace: fp32 [p,p] statistic L~ of the last update */
    SHAMPOO4_BUF_Q = 18,          /* workspace: fp32 [p,p] refreshed eigenvectors Q */
    SHAMPOO4_BUF_ROOT_V = 19,     /* workspace: fp32 [p,p] rectified root eigenvectors of
                                     the last refresh_root (ROOT_CACHE) or precondition */
    SHAMPOO4_BUF_ROOT_MAT = 20,   /* workspace: fp32 [p,p] root matrix V^r diag(d) V^r^T
                                     (ROOT_CACHE: formed at init and at every refresh_root) */
    SHAMPOO4_BUF_STAT64 = 21,     /* workspace, FP64_REFRESH only: fp64 [p,p] statistic L~ */
    SHAMPOO4_BUF_Q64 = 22         /* workspace, FP64_REFRESH only: fp64 [p,p] refreshed Q
                                     (BUF_Q holds it rounded to fp32; with FP64_REFRESH, BUF_V
                                     and BUF_STAT are EINVAL) */
} shampoo4_buffer;

/* ABI version of the loaded library (SHAMPOO4_ABI_VERSION). */
SHAMPOO4_API int32_t shampoo4_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
SHAMPOO4_API const char* shampoo4_strerror(shampoo4_status status);

/* Sizes of the caller-owned buffers for `nblocks` blocks of `shapes` (host array).
 * state_bytes: the optimizer state (codes, scales, eigenvalues, root; serializable).
 * workspace_bytes: descriptor tables, the optional root cache and temporaries.
 * Host only; no HIP call. */
SHAMPOO4_API shampoo4_status shampoo4_plan(const shampoo4_config* cfg, int32_t nblocks,
                              const shampoo4_shape* shapes,
                              size_t* state_bytes, size_t* workspace_bytes);

/* Create a context over caller-owned device buffers (both 256-byte aligned and at
 * least as large as shampoo4_plan reports) and, unless SHAMPOO4_FLAG_KEEP_STATE is
 * set, enqueue the initial state: U = I, lam = 0, root = (I, d = 1) (the pages fix no
 * initial state; the identity root leaves G unchanged until the first refresh).
 * Enqueues the descriptor tables into the workspace and waits for `stream` before
 * returning (init and shampoo4_check are the only calls that synchronize: the host
 * copy of the tables is freed afterwards).  The buffers must outlive the context. */
SHAMPOO4_API shampoo4_status shampoo4_init(const shampoo4_config* cfg, int32_t nblocks,
                              const shampoo4_shape* shapes,
                              void* state, size_t state_bytes,
                              void* workspace, size_t workspace_bytes,
                              void* stream, shampoo4_ctx* out);

/* Diagonal fallback ("Shampoo -- Second-Order Optimizer", "Blocked and distributed
 * variants": if one dimension of a block exceeds a threshold, that side's factor is
 * dropped and diagonal AdaGrad is used along it).  A side marked diagonal keeps no
 * eigenvector matrix: its state is the diagonal of its factor as the same exponential
 * moving average, lam_i <- beta lam_i + (1 - beta) sum_j Gs[i][j]^2 (Gs = G for side L,
 * G^T for side R), updated by update_stats, with d = (lam + eps)^(-1/4) at refresh_root
 * (the same -1/4 exponent as a full side, so the step stays homogeneous of degree 0);
 * precondition uses diag(d) in place of that side's root matrix.  The caller picks the
 * sides (the threshold is the caller's: see blocking.py).  A diagonal side may have an
 * order up to 65536 (a side with eigenvectors: 8192); its state holds no codes and
 * scales (those buffers have size 0 in shampoo4_layout) and it has no workspace
 * matrices (shampoo4_layout of BUF_V .. BUF_ROOT_MAT returns EINVAL). */
#define SHAMPOO4_DIAG_L 1u
#define SHAMPOO4_DIAG_R 2u

/* shampoo4_plan / shampoo4_init with per-block diagonal sides: diag_sides is a host array
 * of nblocks bytes, each SHAMPOO4_DIAG_L | SHAMPOO4_DIAG_R or 0 (NULL: no diagonal side,
 * the plain calls).  EINVAL: other bits; ESHAPE: a dimension above its side's limit. */
SHAMPOO4_API shampoo4_status shampoo4_plan_ex(const shampoo4_config* cfg, int32_t nblocks,
                                              const shampoo4_shape* shapes, const uint8_t* diag_sides,
                                              size_t* state_bytes, size_t* workspace_bytes);
SHAMPOO4_API shampoo4_status shampoo4_init_ex(const shampoo4_config* cfg, int32_t nblocks,
                                              const shampoo4_shape* shapes, const uint8_t* diag_sides,
                                              void* state, size_t state_bytes,
                                              void* workspace, size_t workspace_bytes,
                                              void* stream, shampoo4_ctx* out);

/* One statistics update of every block: io is a host array of nblocks entries
 * (only G/ldg are read).  Per side: the stored eigenvectors are dequantized and
 * rectified ("4-bit Shampoo ..." abstract: the quantized eigenvector matrix is kept and
 * its orthogonality rectified), the factor is rebuilt from them and its eigenvalues and
 * updated with G G^T (side R: G^T G) as an exponential moving average ("Shampoo --
 * Second-Order Optimizer", "Kronecker factorization" for the products, "Pitfalls, and
 * the small-model view" for the EMA), and its eigenpairs are refreshed warm-started
 * from the rectified eigenvectors, L = U Lambda U^T ("Rotation, not just rescaling"),
 * then re-quantized.  The root snapshot is not touched. */
SHAMPOO4_API shampoo4_status shampoo4_update_stats(shampoo4_ctx ctx, const shampoo4_io* io, void* stream);

/* Root refresh of every block: d = (lam + eps)^(-1/4), root codes <- codes.  The
 * damped eigen form of the inverse fourth root, U (Lambda + eps I)^(-1/4) U^T ("Shampoo
 * -- Second-Order Optimizer", "Computing the inverse fourth root"), taken only every
 * T steps while the statistics are updated every step ("The cost dial: update
 * frequency, memory, blocking"); the caller decides when. */
SHAMPOO4_API shampoo4_status shampoo4_refresh_root(shampoo4_ctx ctx, void* stream);

/* Preconditioned direction of every block into io[b].P: L^(-1/4) G R^(-1/4) ("Shampoo
 * -- Second-Order Optimizer", "Where the fourth root comes from") in the eigen form of
 * "Rotation, not just rescaling", with the root eigenvectors dequantized and rectified
 * first ("4-bit Shampoo ..." abstract: rectification also serves the inverse 4-th
 * root).  io[b].G and io[b].P are read / written; G is not modified. */
SHAMPOO4_API shampoo4_status shampoo4_precondition(shampoo4_ctx ctx, const shampoo4_io* io, void* stream);

/* One optimizer step of every block, in the order "Shampoo -- Second-Order Optimizer"
 * gives it: the statistics update every step ("Kronecker factorization"), the inverse
 * roots only when `refresh` is nonzero ("Computing the inverse fourth root"; every T
 * steps, "The cost dial: update frequency, memory, blocking"), then the preconditioned
 * direction into io[b].P ("Where the fourth root comes from"; io as for
 * shampoo4_precondition).  Results
 * equal, bit for bit, those of the three calls above in that order.  Without a refresh
 * and with SHAMPOO4_FLAG_ROOT_CACHE and valid cached roots, the preconditioned direction
 * only reads the cached root matrices and G, so it runs on a second stream of the
 * context (default priority) beside the statistics update; the call makes `stream`
 * wait for it before returning, so later work on `stream` sees P.  Errors as for the
 * three calls; a failed validation enqueues nothing. */
SHAMPOO4_API shampoo4_status shampoo4_step(shampoo4_ctx ctx, const shampoo4_io* io, int32_t refresh, void* stream);

/* Grafting and the weight update ("Shampoo -- Second-Order Optimizer", section
 * "Grafting: borrow a step size that already works"): per block,
 *     W <- W - lr * ||d_graft||_F / (||P||_F + eps_graft) * P
 * with P = io[b].P the preconditioned direction (as written by shampoo4_precondition)
 * and d_graft the step of the grafted method on G = io[b].G:
 *   SHAMPOO4_GRAFT_SGD   d_graft = G;
 *   SHAMPOO4_GRAFT_ADAM  m <- beta1 m + (1 - beta1) G, v <- beta2 v + (1 - beta2) G^2
 *                        (elementwise, moments updated in place),
 *                        d_graft = (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + eps_adam).
 * Norms are block Frobenius norms, reduced in a fixed order (deterministic). */
#define SHAMPOO4_GRAFT_SGD 0
#define SHAMPOO4_GRAFT_ADAM 1

typedef struct {
    int32_t mode;             /* SHAMPOO4_GRAFT_* */
    int32_t step;             /* Adam's step t >= 1 for the bias correction (SGD: ignored) */
    float lr;                 /* eta, finite */
    float eps_graft;          /* >= 0 */
    float beta1, beta2;       /* Adam moment factors in [0, 1) */
    float eps_adam;           /* >= 0 */
} shampoo4_graft_config;

typedef struct {
    float* W;                 /* device, [m, n] weights of the block, row-major, updated in place */
    int64_t ldw;              /* >= n */
    float* M;                 /* device, [m, n] Adam first moment, contiguous (ld n); SGD: unused */
    float* V;                 /* device, [m, n] Adam second moment, contiguous; SGD: unused */
} shampoo4_graft_io;

/* io: G/ldg and P/ldp of every block (read only); gio: nblocks entries.  Two kernels on
 * `stream` (block norms with the Adam moment update, then the scaled update of W).
 * EINVAL: null arguments, a bad mode, a non-finite lr or eps out of range; ESHAPE:
 * ldw < n. */
SHAMPOO4_API shampoo4_status shampoo4_graft(shampoo4_ctx ctx, const shampoo4_io* io, const shampoo4_graft_io* gio,
                                            const shampoo4_graft_config* cfg, void* stream);

/* Wait for `stream`, then report and clear the device non-finite flag
 * (raised when a quantized block or an eigenvalue is NaN/Inf).  *device_flags
 * (may be NULL) receives the raw flag word.  Returns SHAMPOO4_ENONFINITE if set. */
SHAMPOO4_API shampoo4_status shampoo4_check(shampoo4_ctx ctx, void* stream, uint32_t* device_flags);

/* Destroy a context (host memory only; device buffers stay the caller's). */
SHAMPOO4_API shampoo4_status shampoo4_destroy(shampoo4_ctx ctx);

/* Byte offset and size of one per-side buffer inside the state (state buffers,
 * values < 16) or the workspace (values >= 16).  side: 0 = L, 1 = R.  Host only. */
SHAMPOO4_API shampoo4_status shampoo4_layout(shampoo4_ctx ctx, int32_t block, int32_t side,
                                shampoo4_buffer which, size_t* offset, size_t* bytes);

/* Codec in isolation ("4-bit Shampoo ..." abstract: block-wise linear-square 4-bit
 * quantization).  x: device fp32 [n]; codes: device uint8 [ceil(n/64)*32];
 * scales: device fp32 [ceil(n/64)].  Blocks are 64 consecutive elements, the last
 * one zero-padded; element 2i goes to the low nibble of byte i.  qblock must be 64.
 * Non-finite input raises the device flag of no context; the codes are then undefined. */
SHAMPOO4_API shampoo4_status shampoo4_quantize(const float* x, int64_t n, int32_t qblock,
                                  uint8_t* codes, float* scales, void* stream);
SHAMPOO4_API shampoo4_status shampoo4_dequantize(const uint8_t* codes, const float* scales, int64_t n,
                                    int32_t qblock, float* x, void* stream);

/* The float32 codebook the kernels use (host copy): 16 levels (ascending) and the
 * 15 decision midpoints.  Host only. */
SHAMPOO4_API shampoo4_status shampoo4_codebook(float levels[16], float midpoints[15]);

/* The same three calls for a named codebook (SHAMPOO4_CODEBOOK_*; EINVAL otherwise).
 * shampoo4_quantize / shampoo4_dequantize / shampoo4_codebook are these with
 * SHAMPOO4_CODEBOOK_LINEAR_SQUARE. */
SHAMPOO4_API shampoo4_status shampoo4_quantize_ex(const float* x, int64_t n, int32_t qblock, int32_t codebook,
                                                  uint8_t* codes, float* scales, void* stream);
SHAMPOO4_API shampoo4_status shampoo4_dequantize_ex(const uint8_t* codes, const float* scales, int64_t n,
                                                    int32_t qblock, int32_t codebook, float* x, void* stream);
SHAMPOO4_API shampoo4_status shampoo4_codebook_ex(int32_t codebook, float levels[16], float midpoints[15]);

/* Device workspace bytes shampoo4_gemm_batched needs for `count` products. */
SHAMPOO4_API size_t shampoo4_gemm_workspace_bytes(int32_t count);

/* Batched fp32 MFMA GEMM in isolation: for each i < count,
 *   D_i = alpha * op(A_i) op(B_i) + beta * C_i     (op = transpose when trans* != 0)
 * with op(A_i) [M,K], op(B_i) [K,N], C_i and D_i [M,N] row-major.  All pointer arrays
 * are host arrays of device pointers; C may be NULL when beta == 0.  Used to test and
 * time the matrix-product kernels every stage of the step runs on (a 128 x 128 or 64 x 64
 * launch on the three-piece bf16 kernel: see SHAMPOO4_FLAG_FP32_MFMA and
 * shampoo4_gemm_batched_ex).  `workspace` is a
 * 256-byte aligned device buffer of at least shampoo4_gemm_workspace_bytes(count)
 * bytes that receives the descriptors (one host-to-device copy from pageable memory
 * is enqueued before the kernel); it must stay untouched until the kernel ran. */
SHAMPOO4_API shampoo4_status shampoo4_gemm_batched(int32_t count, int32_t transA, int32_t transB,
                                      const int32_t* M, const int32_t* N, const int32_t* K,
                                      float alpha, const float* const* A, const int64_t* lda,
                                      const float* const* B, const int64_t* ldb,
                                      float beta, const float* const* C, const int64_t* ldc,
                                      float* const* D, const int64_t* ldd,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* shampoo4_gemm_batched with a choice of kernel (arguments, workspace and errors as
 * there; EINVAL for another `kernel` value):
 *   SHAMPOO4_GEMM_AUTO  as shampoo4_gemm_batched: the launch's tile shape follows the batch
 *                       (128 x 128 once the products have 512 such tiles, else 64 x 64;
 *                       32-wide tiles for products with a side of at most 32), and a
 *                       128 x 128 or 64 x 64 launch runs on the three-piece bf16 kernel
 *                       (SHAMPOO4_FLAG_FP32_MFMA), with 16-byte loads where every operand
 *                       allows them (16-byte aligned base, pitch and contiguous extent
 *                       multiples of 4), else 4-byte loads;
 *   SHAMPOO4_GEMM_FP32  every product on the fp32 matrix cores;
 *   SHAMPOO4_GEMM_X3    one launch on 128 x 128 tiles whatever the batch, on the three-piece
 *                       bf16 kernel. */
#define SHAMPOO4_GEMM_AUTO 0
#define SHAMPOO4_GEMM_FP32 1
#define SHAMPOO4_GEMM_X3 2
SHAMPOO4_API shampoo4_status shampoo4_gemm_batched_ex(int32_t kernel, int32_t count, int32_t transA, int32_t transB,
                                         const int32_t* M, const int32_t* N, const int32_t* K,
                                         float alpha, const float* const* A, const int64_t* lda,
                                         const float* const* B, const int64_t* ldb,
                                         float beta, const float* const* C, const int64_t* ldc,
                                         float* const* D, const int64_t* ldd,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free form of shampoo4_gemm_batched, for callers that cannot allocate device
 * memory or provide a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, results (bit for bit) and errors as for
 * shampoo4_gemm_batched, without the workspace: the descriptor table goes to a static
 * device array of the library (384 KiB per GPU, held until the process ends; its address
 * is looked up on the first call on each device).  The call allocates no device memory.
 * At most SHAMPOO4_GEMM_STATIC_MAX products per call (more: SHAMPOO4_ESMALLBUF, nothing
 * enqueued).  Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (concurrent streams or host threads) race on it, so order them (one stream, or
 * an event between them).  Nothing in the array needs to start at zero: each call writes
 * the whole table it uses (one copy from pageable host memory, enqueued before the
 * kernel). */
#define SHAMPOO4_GEMM_STATIC_MAX 2048
SHAMPOO4_API shampoo4_status shampoo4_gemm_batched_static(int32_t count, int32_t transA, int32_t transB,
                                             const int32_t* M, const int32_t* N, const int32_t* K,
                                             float alpha, const float* const* A, const int64_t* lda,
                                             const float* const* B, const int64_t* ldb,
                                             float beta, const float* const* C, const int64_t* ldc,
                                             float* const* D, const int64_t* ldd, void* stream);

/* Inverse 4th root by the coupled Newton iteration, matrix products only ("Shampoo --
 * Second-Order Optimizer", section "Computing the inverse fourth root", second route),
 * for the unquantized baseline: for each i < count,
 *     X_i = (A_i + eps I)^(-1/4)
 * with A_i symmetric positive semi-definite [p_i, p_i] (leading dimension lda_i), after
 * scaling by c = ||A_i + eps I||_F: X = I, M = (A_i + eps I) / c, then `iters` times
 * F = (5 I - M) / 4, X <- X F, M <- F^4 M (three grouped MFMA GEMM launches per
 * iteration over all matrices), and X_i = c^(-1/4) X.  M tends to I quadratically once
 * close; a factor with condition number k needs about log(k) / log(2.44) + 5 iterations.
 * Host arrays of device pointers; `workspace` is 256-byte aligned device memory of at
 * least shampoo4_inverse_root_workspace_bytes(count, p) bytes (seven p x p float matrices
 * per input plus descriptor tables, copied from pageable host memory at the call).
 * ESHAPE: p outside 1..8192 or ld < p; EINVAL: null pointers, eps < 0, iters outside
 * 0..100; ESMALLBUF: workspace too small. */
SHAMPOO4_API size_t shampoo4_inverse_root_workspace_bytes(int32_t count, const int32_t* p);
SHAMPOO4_API shampoo4_status shampoo4_inverse_root(int32_t count, const int32_t* p, const float* const* A,
                                                   const int64_t* lda, float eps, int32_t iters,
                                                   float* const* X, const int64_t* ldx,
                                                   void* workspace, size_t workspace_bytes, void* stream);

/* Kernel timing (HIP events around every launch of the next calls on a context).
 * enable != 0 starts recording (clears previous records); the report waits for the
 * device and returns, per kernel family, the number of launches, total milliseconds,
 * and algorithmic flops and bytes.  names: "gemm_bjorck", "gemm_stats", "gemm_power",
 * "gemm_qr", "gemm_qr_trail", "gemm_qr_q", "gemm_rayleigh", "gemm_precond" (the matrix
 * products by the stage they serve; the QR's are split into the products inside an outer
 * reflector block, the block's products on the trailing columns and the accumulation of
 * Q), "dequant", "quant", "qr_panel", "rayleigh", "elementwise", "graft", "diag" (the
 * diagonal sides' statistic and the both-diagonal precondition), "gemm64" (every float64
 * product of FP64_REFRESH), "gemm_x3" (every product that ran on the three-piece bf16
 * kernel, whatever its stage; these are also counted in their stage's family).  Host arrays of
 * length *count (in: capacity, out: used). */
SHAMPOO4_API shampoo4_status shampoo4_timing(shampoo4_ctx ctx, int32_t enable);
SHAMPOO4_API shampoo4_status shampoo4_timing_report(shampoo4_ctx ctx, int32_t* count, const char** names,
                                       int64_t* launches, double* total_ms,
                                       double* flops, double* bytes);

#ifdef __cplusplus
}
#endif

#endif /* SHAMPOO4_H */
