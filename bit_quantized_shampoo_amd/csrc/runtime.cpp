// Host runtime and C ABI of the 4-bit Shampoo step (see include/shampoo4.h).
//
// A context is a static plan: at init every kernel launch of every entry point is
// described once by device descriptor tables (written into the tail of the
// caller's workspace) whose pointers address the caller's state and workspace
// buffers.  G and P change per call, so descriptors refer to them by block index
// into a small io table that is the only thing uploaded per call.  Each entry
// point then just enqueues its fixed sequence of grouped launches on the stream:
// one launch covers every block and both sides of a stage.
#include "../../include/shampoo4.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <memory>
#include <type_traits>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"

#include <rocprofiler-sdk-roctx/roctx.h>

using namespace s4;

namespace {

// A roctx range around each call that enqueues device work: a rocprofv3 run with
// --marker-trace shows the library's calls on the timeline above their kernels (a
// push/pop pair costs nothing measurable when no profiler is attached).
struct CallRange {
    explicit CallRange(const char* name) { roctxRangePushA(name); }
    ~CallRange() { roctxRangePop(); }
    CallRange(const CallRange&) = delete;
    CallRange& operator=(const CallRange&) = delete;
};

}  // namespace

namespace {

constexpr size_t kAlign = 256;
constexpr int kRing = 8;            // pinned io staging slots
static_assert(sizeof(IoEntry) == sizeof(shampoo4_io) && sizeof(GraftIo) == sizeof(shampoo4_graft_io) &&
                  sizeof(GraftIo) == sizeof(IoEntry),
              "per-call tables share the staging slots");
constexpr int kPanel = 32;          // Householder panel width
constexpr int kOuter = 128;         // columns whose reflectors update the trailing matrix together
constexpr int kMaxSplit = GEMM_MAX_SLABS;   // split-K chunks of the skinny QR products
constexpr int kMaxDim = 8192;       // order of a side that keeps eigenvectors
constexpr int kMaxDiagDim = 65536;  // order of a diagonal side

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Timing families: the matrix products are split by the stage they serve.
enum Family {
    FAM_GEMM_BJORCK = 0, FAM_GEMM_STATS, FAM_GEMM_POWER, FAM_GEMM_QR, FAM_GEMM_RAYLEIGH,
    FAM_GEMM_PRECOND, FAM_DEQUANT, FAM_QUANT, FAM_PANEL, FAM_RAYLEIGH, FAM_ELEMENTWISE, FAM_GRAFT,
    FAM_GEMM_QR_TRAIL, FAM_GEMM_QR_Q, FAM_DIAG, FAM_GEMM64, FAM_GEMM_X3, FAM_N
};
// gemm_qr: the reflector products inside an outer block (and the look-ahead schedule's);
// gemm_qr_trail: an outer block's reflectors on the trailing columns; gemm_qr_q: the
// accumulation of Q; gemm_x3: every product that ran on the three-piece bf16 kernel,
// whatever its stage (also counted in its stage's family)
const char* kFamilyNames[FAM_N] = {"gemm_bjorck", "gemm_stats", "gemm_power", "gemm_qr", "gemm_rayleigh",
                                   "gemm_precond", "dequant", "quant", "qr_panel", "rayleigh",
                                   "elementwise", "graft", "gemm_qr_trail", "gemm_qr_q", "diag", "gemm64",
                                   "gemm_x3"};

enum Kind { K_GEMM, K_DEQUANT, K_QUANT, K_COPY, K_PANEL, K_RAYLEIGH, K_ROOT, K_IDENTITY, K_SIGN, K_INIT,
            K_RECORD, K_WAIT, K_GRAFT_NORMS, K_GRAFT_APPLY, K_COPYF, K_NEWTON_NORM, K_NEWTON_SCALE,
            K_NEWTON_ELEM, K_QRSTEP, K_DIAG_PARTIALS, K_DIAG_EMA, K_DIAG_SCALE, K_GEMM64, K_PANEL64,
            K_COLDOT64, K_IDENT64, K_CVT };

struct Launch {
    Kind kind = K_GEMM;
    int cfg = 0;
    int mode = 0;        // GEMM: shared transpose flags or GEMM_MODE_MIXED; panel, QR step: rows class;
                         // identity fill: 1 = diag(sign(R_jj))
    int fam = FAM_ELEMENTWISE;
    size_t desc_off = 0, prefix_off = 0;   // offsets inside the descriptor region (QR step: the
                                           // panel table and the slab table)
    int ndesc = 0, ntiles = 0, max_h = 0;
    int strm = 0;        // 0: the caller's stream, 1: the context's second stream
    bool vec = false;    // GEMM: 16-byte operand loads (io operands: also checked per call)
    bool slab = false;   // GEMM: some operand sums split-K slabs
    bool kscale = false; // GEMM: some product scales op(B)'s rows
    bool uses_io = false;
    bool f32in = false;  // fp64 GEMM: float operands (the gradients)
    int ev = -1;         // K_RECORD / K_WAIT: index of the context's synchronization event
    double flops = 0, bytes = 0;
};
using Seq = std::vector<Launch>;

struct Side {
    int p = 0, q = 0;
    bool diag = false;   // diagonal fallback: only the diagonal statistic (lam) and d
    int64_t nqb = 0;
    // state offsets
    size_t codes = 0, scales = 0, lam = 0, rcodes = 0, rscales = 0, d = 0;
    // workspace offsets
    size_t Vs = 0, Vr = 0, Tmp = 0, Wg = 0, Lt = 0, Pm = 0, Qm = 0, Vb = 0, Yb = 0, Z = 0, W = 0, Mb = 0,
           Z2 = 0, rdiag = 0, Tb = 0, Rt = 0;
    // float64 statistics update: Bjorck ping-pong, Gram, statistic, P (factored in place), Q,
    // the panels' V and Y, the trailing / Q products' intermediates and R's diagonal
    size_t V64a = 0, V64b = 0, Wg64 = 0, Lt64 = 0, P64 = 0, Q64 = 0, Vb64 = 0, Yb64 = 0, Z64 = 0, W64 = 0,
           rd64 = 0;
    std::vector<size_t> outer_rows;   // row offset of outer block o inside Vb / Yb (pitch = outer width)
};

struct TimingRec {
    int family;
    bool x3;             // a matrix product on the three-piece bf16 kernel
    hipEvent_t e0, e1;
    double flops, bytes;
};

}  // namespace

struct shampoo4_ctx_s {
    shampoo4_config cfg{};
    int nb = 0;
    std::vector<shampoo4_shape> shapes;
    uint8_t* st = nullptr;
    uint8_t* ws = nullptr;
    size_t st_bytes = 0, ws_bytes = 0;
    std::vector<Side> sides;             // 2 per block: L then R
    std::vector<std::reference_wrapper<Side>> full;   // the sides that keep eigenvectors
    std::vector<uint8_t> diag_bits;      // per block: SHAMPOO4_DIAG_L | SHAMPOO4_DIAG_R
    std::vector<size_t> X1, X2;          // per block precondition temporaries
    std::vector<size_t> RP, CP;          // per block partial row / column sums of G^2 (diagonal sides)
    size_t io_off = 0, gio_off = 0, flag_off = 0, parts_off = 0, desc_base = 0;
    std::vector<uint8_t> last_io, last_gio;   // host copies of the tables last uploaded
    std::vector<uint8_t> blob;           // descriptor region contents
    size_t lds_limit = 0;                // bytes of LDS one workgroup may use
    int max_panels = 0;

    Seq deq_stats, deq_root, init_seq;
    std::vector<Seq> bj_stats, bj_root;
    Seq stats_x[2], stats_g, power_first[2], power_next;
    // statistics with (1 - beta) G G^T folded into the first Bjorck Gram launch (which
    // does not fill the GPU by itself) and beta V diag(lam) V^T added onto it
    std::vector<Seq> bj_stats_fold;
    Seq stats_x_fold;
    std::vector<Seq> qr_steps;            // per panel index: panel, block and trailing products
    Seq qr_join;                          // second stream's work joined back (look-ahead plans)
    int outer = kOuter;                   // columns whose reflectors update the trailing matrix together
    bool lookahead = false;               // small batches: trailing and Q updates on a second stream
    bool fused = false;                   // small batches: one launch per panel (QR step kernel)
    bool qr_split = false;                // blocked QR of two groups of sides on two streams
    bool fp32_state = false;              // U kept in float32 (the 32-bit baseline), no codec
    bool fp64 = false;                    // statistics update in float64 (FP64_REFRESH)
    Seq s64_pre, s64_stats, s64_power_first, s64_power_next, s64_qinit, s64_post;   // float64 update
    std::vector<Seq> s64_bjorck, s64_qr, s64_qacc;
    int codebook = SHAMPOO4_CODEBOOK_LINEAR_SQUARE;   // 4-bit codebook of U and the root
    int n_sync = 0;                       // synchronization events the plan uses
    hipStream_t aux = nullptr;
    // precondition overlapped with the statistics update (shampoo4_step): its stream and
    // the fork / join events, created on first use
    hipStream_t pre_strm = nullptr;
    hipEvent_t pre_fork = nullptr, pre_join = nullptr;
    std::vector<hipEvent_t> sync_ev;
    // update_stats replayed from a HIP graph (captured on `cap` at the first call of each
    // variant: with or without the cached rectified eigenvectors, and with or without
    // 16-byte loads of the gradients, which the captured kernels bake in)
    bool use_graphs = false;
    bool x3 = true;                       // 128 x 128 and 64 x 64 products on the three-piece bf16 kernel
    // SHAMPOO4_FLAG_DEBUG: workspace temporaries (offset, bytes), filled with NaN before each
    // call; a descriptor found reaching outside the state or workspace at init
    bool debug = false;
    std::vector<std::pair<size_t, size_t>> temps;
    bool bad_desc = false;
    bool graph_ok = true;
    hipStream_t cap = nullptr;
    hipGraphExec_t stats_graph[2][2] = {};
    Seq qinit, sign, ray_gemm, rayleigh, quant, root_d, root_copy;
    Seq qinit_signed;                     // backward accumulation: Q starts as diag(sign(R_jj))
    Seq pre[4];
    Seq root_mat, pre_cached[2];        // ROOT_CACHE: root matrices, then two products per block
    // the same two products on 128 x 128 tiles, for the copy beside the QR chain: fewer,
    // longer workgroups leave most CUs to the panel launches
    Seq pre_side[2];
    Seq graft_seq[2];                    // per graft mode (bytes differ): norms, apply
    Seq diag_stats, diag_pre;            // diagonal sides: statistic; P of blocks with both sides diagonal
    GraftParams graft_prm{};
    float newton_eps = 0.f;              // damping of the coupled Newton inverse root (standalone call)

    bool root_v_valid = false;        // workspace Vr holds Bjorck(dequant(root codes))
    bool root_v_is_stats = false;     // ... and the root codes equal the current codes

    // io staging
    uint8_t* pinned = nullptr;
    bool io_vec = false;              // every G of the current call allows 16-byte loads
    hipEvent_t ring_ev[kRing] = {};
    bool ring_used[kRing] = {};
    int ring_next = 0;

    // timing
    bool timing = false;
    std::vector<TimingRec> recs;
    std::vector<hipEvent_t> ev_pool;
    size_t ev_used = 0;

    ~shampoo4_ctx_s() {
        for (auto& e : ring_ev)
            if (e) (void)hipEventDestroy(e);
        for (auto& e : ev_pool) (void)hipEventDestroy(e);
        for (auto& e : sync_ev)
            if (e) (void)hipEventDestroy(e);
        for (auto& gv : stats_graph)
            for (auto& g : gv)
                if (g) (void)hipGraphExecDestroy(g);
        if (aux) (void)hipStreamDestroy(aux);
        if (pre_strm) (void)hipStreamDestroy(pre_strm);
        if (pre_fork) (void)hipEventDestroy(pre_fork);
        if (pre_join) (void)hipEventDestroy(pre_join);
        if (cap) (void)hipStreamDestroy(cap);
        if (pinned) (void)hipHostFree(pinned);
    }

    template <class T>
    T* wsp(size_t off) const { return reinterpret_cast<T*>(ws + off); }
    template <class T>
    T* stp(size_t off) const { return reinterpret_cast<T*>(st + off); }
    float* wsf(size_t off) const { return wsp<float>(off); }
    float* stf(size_t off) const { return stp<float>(off); }

    // ---- debug checks (SHAMPOO4_FLAG_DEBUG) -------------------------------------
    // [p, p + bytes) must lie inside the state or the workspace's data region (below the
    // descriptor tables); a null pointer or an empty extent passes.
    void check_range(const void* p, int64_t bytes) {
        if (!debug || !p || bytes <= 0 || !ws) return;
        const uint8_t* q = static_cast<const uint8_t*>(p);
        const bool in_ws = q >= ws && q + bytes <= ws + desc_base;
        const bool in_st = st && q >= st && q + bytes <= st + st_bytes;
        if (!in_ws && !in_st) bad_desc = true;
    }
    // bytes spanned by a rows x cols float matrix of pitch ld (plus nslab - 1 slabs of
    // `slab` elements after it)
    static int64_t span(int64_t rows, int64_t cols, int64_t ld, int64_t nslab = 1, int64_t slab = 0,
                        int64_t elem = 4) {
        if (rows <= 0 || cols <= 0) return 0;
        return ((rows - 1) * ld + cols + std::max<int64_t>(nslab - 1, 0) * slab) * elem;
    }
    void check_gemm(const GemmDesc& d, bool ta, bool tb) {
        if (!debug) return;
        if (d.a_io < 0) check_range(d.A, span(ta ? d.K : d.M, ta ? d.M : d.K, d.lda, d.anslab, d.aslab));
        if (d.b_io < 0) check_range(d.B, span(tb ? d.N : d.K, tb ? d.K : d.N, d.ldb, d.bnslab, d.bslab));
        const bool coldot = d.flags & GEMM_F_COLDOT;
        if (d.beta != 0.f || coldot) check_range(d.C, span(d.M, d.N, d.ldc));
        if (d.d_io < 0) {
            const int64_t rows = coldot ? (d.M + 127) / 128 : d.M;   // column-dot: one row per tile (at most)
            check_range(d.D, span(rows, d.N, d.ldd, std::max(1, d.ksplit), d.dslab));
        }
        check_range(d.kscale, (int64_t)d.K * 4);
        check_range(d.rscale, (int64_t)d.M * 4);
        check_range(d.cscale, (int64_t)d.N * 4);
    }
    void check_codec(const CodecDesc& d) {
        if (!debug) return;
        const int64_t nb = (d.n + 63) / 64;
        check_range(d.codes_in, nb * 32);
        check_range(d.scales_in, nb * 4);
        check_range(d.codes_out, nb * 32);
        check_range(d.scales_out, nb * 4);
        check_range(d.x_in, d.n * 4);
        check_range(d.x_out, d.n * 4);
    }
    // NaN into every temporary (a kernel that reads one before writing it then yields NaN)
    hipError_t debug_fill(hipStream_t s) {
        if (!debug) return hipSuccess;
        for (auto& t : temps) {
            hipError_t e = hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(ws + t.first), 0x7fc00000,
                                             t.second / 4, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }

    // ---- descriptor region ---------------------------------------------------
    size_t blob_put(const void* data, size_t bytes) {
        const size_t off = align_up(blob.size());
        blob.resize(off + align_up(bytes ? bytes : 1), 0);
        if (bytes) std::memcpy(blob.data() + off, data, bytes);
        return off;
    }

    struct GemmItem {
        GemmDesc d;
        bool ta, tb;
    };

    // Tile shape that wastes least of its tile on a product: skinny products (one side
    // up to 32, the panel-wide reflector products) take the 32-wide tiles, products with a
    // side up to 64 the 64 x 64 tile; -1: square enough for either of the large shapes.
    static int shape_class(const GemmDesc& d) {
        if (d.M <= 32) return GEMM_32x128;
        if (d.N <= 32) return GEMM_128x32;
        if (d.M <= 64 || d.N <= 64) return GEMM_64x64;
        return -1;
    }
    // Multiply-adds a tile shape computes for a product, padding included.
    static double padded_work(const GemmDesc& d, int cfg) {
        int bm, bn;
        gemm_tile_dims(cfg, &bm, &bn);
        return (double)((d.M + bm - 1) / bm * bm) * ((d.N + bn - 1) / bn * bn) * d.K;
    }
    // The large-shape choice for a set of products: 128 x 128 when its tiles fill the
    // GPU's workgroup slots (two per CU), else 64 x 64; products of at most 32 rows
    // always take the 32 x 128 tile.
    static int default_cfg(const std::vector<GemmItem>& items) {
        int maxM = 0;
        long tiles128 = 0;
        for (auto& it : items) {
            const GemmDesc& d = it.d;
            if (d.M <= 0 || d.N <= 0) continue;
            maxM = std::max(maxM, d.M);
            const long t = (d.M + 127) / 128;
            const bool sym = (d.flags & GEMM_F_SYM) && d.M == d.N;
            tiles128 += sym ? t * (t + 1) / 2 : t * ((d.N + 127) / 128);
        }
        return maxM <= 32 ? GEMM_32x128 : (tiles128 >= 512 ? GEMM_128x128 : GEMM_64x64);
    }

    // Launches for a batch of products (mixed transposes allowed).
    // With split_modes, products of different transpose modes go to separate launches
    // of the specialized kernels (fewer registers than the mixed kernel, which spills a
    // little at the 128 x 128 tile).  With by_shape, products are grouped by tile shape
    // class (one launch each) when the padding this saves outweighs the extra launches;
    // otherwise one launch covers them all.  Products with a column-dot epilogue stay in
    // one launch (their partial rows follow one tile height).  groups (optional): the
    // products of each launch, in launch order.
    Seq make_gemm(std::vector<GemmItem> items, int fam, bool split_modes = false, bool by_shape = true,
                  std::vector<std::vector<GemmItem>>* groups = nullptr) {
        auto launch_one = [&](const std::vector<GemmItem>& part, int cfgsel) {
            Seq g = gemm_launch(part, fam, cfgsel);
            if (groups && !g.empty()) groups->push_back(part);
            return g;
        };
        if (split_modes) {
            Seq out;
            for (int mode = 0; mode < 4; ++mode) {
                std::vector<GemmItem> part;
                for (auto& it : items)
                    if (((it.ta ? GEMM_F_TA : 0) | (it.tb ? GEMM_F_TB : 0)) == mode) part.push_back(it);
                if (part.empty()) continue;
                Seq g = make_gemm(part, fam, false, by_shape, groups);
                out.insert(out.end(), g.begin(), g.end());
            }
            return out;
        }
        bool coldot = false;
        for (auto& it : items) coldot = coldot || (it.d.flags & GEMM_F_COLDOT);
        if (by_shape && !coldot) {
            std::vector<GemmItem> part[GEMM_NCFG + 1];   // by class; the last: square
            for (auto& it : items) {
                if (it.d.M <= 0 || it.d.N <= 0) continue;
                const int c = shape_class(it.d);
                part[c < 0 ? GEMM_NCFG : c].push_back(it);
            }
            int nclass = 0;
            for (auto& pt : part) nclass += !pt.empty();
            if (nclass > 1) {
                // one launch: every product on the batch's default shape; grouped: each
                // class on its own shape.  A launch is worth about 5 us of padded work at
                // 80 TFLOP/s.
                const double launch_work = 5e-6 * 80e12 / 2;
                const int c1 = default_cfg(items);
                double one = launch_work, grouped = 0;
                for (int c = 0; c <= GEMM_NCFG; ++c) {
                    if (part[c].empty()) continue;
                    const int cc = c < GEMM_NCFG ? c : default_cfg(part[c]);
                    grouped += launch_work;
                    for (auto& it : part[c]) {
                        one += padded_work(it.d, c1);
                        grouped += padded_work(it.d, cc);
                    }
                }
                if (grouped < one) {
                    Seq out;
                    for (int c = 0; c <= GEMM_NCFG; ++c) {
                        if (part[c].empty()) continue;
                        Seq g = launch_one(part[c], c < GEMM_NCFG ? c : default_cfg(part[c]));
                        out.insert(out.end(), g.begin(), g.end());
                    }
                    return out;
                }
            } else if (nclass == 1) {
                for (int c = 0; c < GEMM_NCFG; ++c)
                    if (!part[c].empty()) return launch_one(part[c], c);
            }
        }
        return launch_one(items, default_cfg(items));
    }

    // One launch of `items` on tile shape cfgsel (128 x 128 and 64 x 64: on the three-piece
    // bf16 kernel unless allow_x3 is false or the context keeps the fp32 matrix cores).
    Seq gemm_launch(const std::vector<GemmItem>& items, int fam, int cfgsel, bool allow_x3 = true) {
        std::vector<GemmDesc> ds;
        int modes = 0, first_mode = -2;
        for (auto& it : items) {
            if (it.d.M <= 0 || it.d.N <= 0) continue;
            GemmDesc d = it.d;
            d.flags = (d.flags & ~(GEMM_F_TA | GEMM_F_TB)) | (it.ta ? GEMM_F_TA : 0) | (it.tb ? GEMM_F_TB : 0);
            const int m = d.flags & (GEMM_F_TA | GEMM_F_TB);
            if (first_mode == -2) first_mode = m;
            if (m != first_mode) modes = 1;
            ds.push_back(d);
        }
        if (ds.empty()) return {};
        // the three-piece bf16 kernel takes the 128 x 128 and 64 x 64 launches without
        // split-K slab sums
        bool slab = false;
        for (auto& d : ds) slab = slab || d.anslab > 1 || d.bnslab > 1;
        if (x3 && allow_x3 && !slab) {
            if (cfgsel == GEMM_128x128) cfgsel = GEMM_X3;
            else if (cfgsel == GEMM_64x64) cfgsel = GEMM_X3_64;
        }
        int bm, bn;
        gemm_tile_dims(cfgsel, &bm, &bn);
        // a symmetric product computes the tiles on and above the diagonal (square tiles,
        // no row / column scales)
        for (auto& d : ds)
            if (bm != bn || d.M != d.N || d.rscale || d.cscale || (d.flags & GEMM_F_COLDOT))
                d.flags &= ~GEMM_F_SYM;
        std::vector<int> prefix;
        int total = 0;
        Launch L;
        for (auto& d : ds) {
            d.tiles_m = (d.M + bm - 1) / bm;
            check_gemm(d, d.flags & GEMM_F_TA, d.flags & GEMM_F_TB);
            prefix.push_back(total);
            if (d.flags & GEMM_F_SYM) {
                const int t = d.tiles_m;
                total += t * (t + 1) / 2 * std::max(1, d.ksplit);
                // algorithmic work of a symmetric product: its M (M + 1) / 2 distinct entries
                L.flops += (double)d.M * (d.M + 1) * d.K;
            } else {
                total += d.tiles_m * ((d.N + bn - 1) / bn) * std::max(1, d.ksplit);
                L.flops += 2.0 * d.M * d.N * d.K;
            }
            const bool coldot = d.flags & GEMM_F_COLDOT;
            L.bytes += 4.0 * ((double)d.M * d.K + (double)d.K * d.N +
                              (double)d.M * d.N * ((d.beta != 0.f || coldot) ? 2 : 1));
        }
        prefix.push_back(total);
        L.vec = true;
        for (auto& d : ds) {
            L.vec = L.vec && gemm_vec_ok(d);
            L.slab = L.slab || d.anslab > 1 || d.bnslab > 1;
            L.kscale = L.kscale || d.kscale != nullptr;
            L.uses_io = L.uses_io || d.a_io >= 0 || d.b_io >= 0;
        }
        L.kind = K_GEMM;
        L.fam = fam;
        L.cfg = cfgsel;
        // a 64 x 64 launch of at most four tiles per CU runs its tiles with two K groups
        // of waves (two waves per SIMD where one tile per CU would give one)
        if (cfgsel == GEMM_64x64 && L.vec && !L.slab && total <= 1024) L.cfg = GEMM_64x64_K2;
        L.mode = modes ? GEMM_MODE_MIXED : first_mode;
        L.ndesc = (int)ds.size();
        L.ntiles = total;
        L.desc_off = blob_put(ds.data(), ds.size() * sizeof(GemmDesc));
        L.prefix_off = blob_put(prefix.data(), prefix.size() * sizeof(int));
        return {L};
    }

    template <class D>
    Launch make_items(Kind kind, const std::vector<D>& ds, const std::vector<int>& tiles) {
        if constexpr (std::is_same_v<D, CodecDesc>)
            for (auto& d : ds) check_codec(d);
        Launch L;
        L.kind = kind;
        L.fam = kind == K_DEQUANT ? FAM_DEQUANT : kind == K_QUANT ? FAM_QUANT : kind == K_PANEL ? FAM_PANEL
              : kind == K_RAYLEIGH ? FAM_RAYLEIGH
              : (kind == K_GRAFT_NORMS || kind == K_GRAFT_APPLY) ? FAM_GRAFT
              : (kind == K_DIAG_PARTIALS || kind == K_DIAG_EMA || kind == K_DIAG_SCALE) ? FAM_DIAG
              : FAM_ELEMENTWISE;
        std::vector<int> prefix;
        int total = 0;
        for (int t : tiles) {
            prefix.push_back(total);
            total += t;
        }
        prefix.push_back(total);
        L.ndesc = (int)ds.size();
        L.ntiles = total;
        L.desc_off = blob_put(ds.data(), ds.size() * sizeof(D));
        L.prefix_off = blob_put(prefix.data(), prefix.size() * sizeof(int));
        return L;
    }

    // ---- plan ---------------------------------------------------------------------
    void layout() {
        fp32_state = (cfg.flags & SHAMPOO4_FLAG_FP32_STATE) != 0;
        fp64 = (cfg.flags & SHAMPOO4_FLAG_FP64_REFRESH) != 0;
        codebook = (cfg.flags & SHAMPOO4_FLAG_DT_CODEBOOK) ? SHAMPOO4_CODEBOOK_DYNAMIC_TREE
                                                           : SHAMPOO4_CODEBOOK_LINEAR_SQUARE;
        use_graphs = (cfg.flags & SHAMPOO4_FLAG_GRAPHS) != 0;
        x3 = (cfg.flags & SHAMPOO4_FLAG_FP32_MFMA) == 0;
        debug = (cfg.flags & SHAMPOO4_FLAG_DEBUG) != 0;
        temps.clear();
        // Large batches are throughput-bound: reflectors go to the trailing matrix 128
        // columns at a time.  Small ones are bound by the chain of panels and by launch
        // latency: panel-wide updates on the caller's stream (or, on request, with the
        // trailing and Q updates overlapped on a second stream).
        double work = 0;
        int max_order = 0;
        for (int b = 0; b < nb; ++b) {
            const double m = shapes[b].m, n = shapes[b].n;
            if (!(diag_bits[b] & SHAMPOO4_DIAG_L)) { work += m * m * m; max_order = std::max(max_order, shapes[b].m); }
            if (!(diag_bits[b] & SHAMPOO4_DIAG_R)) { work += n * n * n; max_order = std::max(max_order, shapes[b].n); }
        }
        lookahead = (cfg.flags & SHAMPOO4_FLAG_QR_LOOKAHEAD) != 0;
        const bool blocked = (cfg.flags & SHAMPOO4_FLAG_QR_BLOCKED) ||
                             (!lookahead && work >= 16.0 * 1073741824.0);
        // the float64 QR goes panel by panel; orders from 2048 take outer blocks of twice the
        // width (half the passes of the trailing and Q updates over the matrix; measured
        // +1.9% on 64 blocks of 4096, -1.6% and -2% on batches of orders up to 1024)
        outer = (blocked && !fp64) ? (max_order >= 2048 ? 2 * kOuter : kOuter) : kPanel;
        // two streams for the blocked QR of batches of orders below 2048 (measured +2.5% on
        // 288 blocks of 1024, +3.2% on the 154-block conv batch; on 64 blocks of 4096 the
        // tall panels in global memory lose to the other group's products what the overlap
        // gains: -0.7%)
        qr_split = blocked && !fp64 && !lookahead && nb >= 2 && max_order < 2048;
        sides.assign(2 * nb, Side{});
        size_t so = 0, wo = 0;
        auto st_take = [&](size_t b) { size_t o = so; so += align_up(b ? b : 1); return o; };
        auto ws_take = [&](size_t b) { size_t o = wo; wo += align_up(b ? b : 1); return o; };
        // a buffer written before it is read within every call (none survives to the next)
        auto tmp_take = [&](size_t b) {
            const size_t o = ws_take(b);
            if (b) temps.emplace_back(o, b);
            return o;
        };
        io_off = ws_take((size_t)nb * sizeof(IoEntry));
        gio_off = ws_take((size_t)nb * sizeof(GraftIo));
        flag_off = ws_take(sizeof(uint32_t) * 4);
        {   // grafting partials: two floats per row tile of every block
            size_t tiles = 0;
            for (auto& sh : shapes) tiles += (sh.m + graft_rows(sh.n) - 1) / graft_rows(sh.n);
            parts_off = tmp_take(tiles * 2 * sizeof(float));
        }
        X1.resize(nb);
        X2.resize(nb);
        RP.assign(nb, 0);
        CP.assign(nb, 0);
        for (int b = 0; b < nb; ++b) {
            for (int s = 0; s < 2; ++s) {
                Side& S = sides[2 * b + s];
                S.p = s == 0 ? shapes[b].m : shapes[b].n;
                S.q = s == 0 ? shapes[b].n : shapes[b].m;
                S.diag = (diag_bits[b] & (s == 0 ? SHAMPOO4_DIAG_L : SHAMPOO4_DIAG_R)) != 0;
                const int64_t p = S.p;
                if (S.diag) {   // the diagonal statistic and d only
                    S.nqb = 0;
                    S.codes = st_take(0);
                    S.scales = st_take(0);
                    S.lam = st_take(p * 4);
                    S.rcodes = st_take(0);
                    S.rscales = st_take(0);
                    S.d = st_take(p * 4);
                    continue;
                }
                S.nqb = (p * p + 63) / 64;
                const size_t ubytes = fp32_state ? (size_t)p * p * 4 : (size_t)S.nqb * 32;
                const size_t sbytes = fp32_state ? 0 : (size_t)S.nqb * 4;
                S.codes = st_take(ubytes);
                S.scales = st_take(sbytes);
                S.lam = st_take(p * 4);
                S.rcodes = st_take(ubytes);
                S.rscales = st_take(sbytes);
                S.d = st_take(p * 4);
                const size_t mat = (size_t)p * p * 4;
                if (fp64) {   // float32: dequantized U, the root and Q for the quantizer only
                    S.Vr = ws_take(mat);
                    S.Rt = ws_take(mat);
                    S.Tmp = tmp_take(mat);
                    S.Wg = tmp_take(mat);
                    S.Qm = tmp_take(mat);
                    const size_t mat64 = (size_t)p * p * 8;
                    S.V64a = tmp_take(mat64);
                    S.V64b = tmp_take(mat64);
                    S.Wg64 = tmp_take(mat64);
                    S.Lt64 = tmp_take(mat64);
                    S.P64 = tmp_take(mat64);
                    S.Q64 = tmp_take(mat64);
                    S.outer_rows.clear();
                    size_t rows = 0;
                    for (int c0 = 0; c0 < p; c0 += kPanel) {
                        S.outer_rows.push_back(rows);
                        rows += p - c0;
                    }
                    S.Vb64 = tmp_take(rows * kPanel * 8);
                    S.Yb64 = tmp_take(rows * kPanel * 8);
                    S.Z64 = tmp_take((size_t)kPanel * p * 8);
                    S.W64 = tmp_take((size_t)kPanel * p * 8);
                    S.rd64 = tmp_take((size_t)p * 8);
                    continue;
                }
                S.Vs = tmp_take(mat);
                S.Vr = ws_take(mat);   // rectified root eigenvectors (kept between calls)
                S.Rt = ws_take(mat);   // root matrix V^r diag(d) V^r^T (ROOT_CACHE)
                S.Tmp = tmp_take(mat);
                S.Wg = tmp_take(mat);
                S.Lt = tmp_take(mat);
                S.Pm = tmp_take(mat);
                S.Qm = tmp_take(mat);
                S.outer_rows.clear();
                size_t rows = 0;
                for (int c0 = 0; c0 < p; c0 += outer) {
                    S.outer_rows.push_back(rows);
                    rows += p - c0;
                }
                S.Vb = tmp_take(rows * outer * 4);
                S.Yb = tmp_take(rows * outer * 4);
                S.Z = tmp_take((size_t)kMaxSplit * outer * p * 4);        // split-K slabs of Y^T A
                S.W = tmp_take((size_t)kMaxSplit * outer * p * 4);        // split-K slabs of Q Y
                S.Mb = tmp_take((size_t)kMaxSplit * outer * kPanel * 4);  // split-K slabs of V^T Y
                S.Z2 = tmp_take((size_t)kMaxSplit * kPanel * kPanel * 4); // look-ahead Y^T A
                S.rdiag = tmp_take(p * 4);
                S.Tb = tmp_take((size_t)((p + kPanel - 1) / kPanel) * kPanel * kPanel * 4);   // fused QR: T per panel
            }
            X1[b] = tmp_take((size_t)shapes[b].m * shapes[b].n * 4);
            X2[b] = tmp_take((size_t)shapes[b].m * shapes[b].n * 4);
            const int64_t m = shapes[b].m, n = shapes[b].n;
            if (diag_bits[b] & SHAMPOO4_DIAG_L) RP[b] = tmp_take((size_t)((n + DIAG_TC - 1) / DIAG_TC) * m * 4);
            if (diag_bits[b] & SHAMPOO4_DIAG_R) CP[b] = tmp_take((size_t)((m + DIAG_TR - 1) / DIAG_TR) * n * 4);
        }
        st_bytes = so;
        desc_base = wo;
        max_panels = 0;
        full.clear();
        for (auto& S : sides)
            if (!S.diag) {
                full.push_back(S);
                max_panels = std::max(max_panels, (S.p + kPanel - 1) / kPanel);
            }
    }

    GemmDesc gd(const float* A, int64_t lda, const float* B, int64_t ldb, float* D, int64_t ldd,
                int M, int N, int K, float alpha = 1.f, float beta = 0.f, const float* C = nullptr,
                int64_t ldc = 0) const {
        GemmDesc d;
        std::memset(&d, 0, sizeof(d));
        d.A = A; d.B = B; d.C = C; d.D = D;
        d.lda = lda; d.ldb = ldb; d.ldc = ldc ? ldc : ldd; d.ldd = ldd;
        d.M = M; d.N = N; d.K = K;
        d.alpha = alpha; d.beta = beta;
        d.a_io = d.b_io = d.d_io = -1;
        return d;
    }

    // Bjorck chain for one family of buffers; the result lands in `fin`.
    static VecDesc copyf_desc(const float* src, float* dst, int64_t n) {
        VecDesc v;
        std::memset(&v, 0, sizeof(v));
        v.a = src;
        v.out = dst;
        v.ld = n;   // element count
        return v;
    }
    static int copyf_tiles(int64_t n) { return (int)((n + COPYF_TILE - 1) / COPYF_TILE); }

    // gram0_extra: products that ride in the first iteration's Gram launch
    void build_bjorck(bool root, Seq& deq, std::vector<Seq>& iters,
                      const std::vector<GemmItem>* gram0_extra = nullptr) {
        const int k = cfg.bjorck_iters;
        std::vector<CodecDesc> cds;
        std::vector<int> tiles;
        for (Side& S : full) {
            const size_t fin = root ? S.Vr : S.Vs;
            const size_t start = (k % 2 == 1) ? S.Tmp : fin;
            CodecDesc c;
            std::memset(&c, 0, sizeof(c));
            c.codes_in = stp<uint8_t>(root ? S.rcodes : S.codes);
            c.scales_in = stf(root ? S.rscales : S.scales);
            c.x_out = wsf(start);
            c.n = (int64_t)S.p * S.p;
            cds.push_back(c);
            tiles.push_back((int)dequant_tiles(c.n));
        }
        if (fp32_state) {   // 32-bit state: U is copied into the Bjorck chain's first buffer
            std::vector<VecDesc> vd;
            std::vector<int> vt;
            for (Side& S : full) {
                const size_t fin = root ? S.Vr : S.Vs;
                vd.push_back(copyf_desc(stf(root ? S.rcodes : S.codes), wsf((k % 2 == 1) ? S.Tmp : fin),
                                        (int64_t)S.p * S.p));
                vt.push_back(copyf_tiles(vd.back().ld));
            }
            Launch L = make_items(K_COPYF, vd, vt);
            L.fam = FAM_DEQUANT;
            for (Side& S : full) L.bytes += (double)S.p * S.p * 8.0;
            deq = {L};
        } else {
            Launch L = make_items(K_DEQUANT, cds, tiles);
            for (Side& S : full) L.bytes += (double)S.p * S.p * (4.0 + 0.5 + 4.0 / 64);
            deq = {L};
        }
        iters.clear();
        for (int i = 0; i < k; ++i) {
            std::vector<GemmItem> gram, upd;
            for (Side& S : full) {
                const size_t fin = root ? S.Vr : S.Vs;
                const size_t start = (k % 2 == 1) ? S.Tmp : fin;
                const size_t other = (start == S.Tmp) ? fin : S.Tmp;
                const size_t in = (i % 2 == 0) ? start : other;
                const size_t out = (i % 2 == 0) ? other : start;
                const int p = S.p;
                GemmDesc gw = gd(wsf(in), p, wsf(in), p, wsf(S.Wg), p, p, p, p);
                gw.flags |= GEMM_F_SYM;                  // V^T V
                gram.push_back({gw, true, false});
                upd.push_back({gd(wsf(in), p, wsf(S.Wg), p, wsf(out), p, p, p, p, -0.5f, 1.5f, wsf(in), p),
                               false, false});
            }
            if (i == 0 && gram0_extra) gram.insert(gram.end(), gram0_extra->begin(), gram0_extra->end());
            Seq s = make_gemm(gram, FAM_GEMM_BJORCK);
            Seq u = make_gemm(upd, FAM_GEMM_BJORCK);
            s.insert(s.end(), u.begin(), u.end());
            iters.push_back(s);
        }
    }

    // ---- Householder QR ---------------------------------------------------------
    static long tiles64(long M, long N) { return ((M + 63) / 64) * ((N + 63) / 64); }
    // split-K factor for a launch whose products have `tiles` 64 x 64 output tiles and
    // depth at least min_k: a batch too small to fill the GPU still spreads its long-K
    // (K = panel height) products
    static int split_for(long tiles, int min_k) {
        if (tiles <= 0 || tiles >= 512) return 1;
        const int ks = (int)std::min<long>(kMaxSplit, (512 + tiles - 1) / tiles);
        return std::max(1, std::min(ks, min_k / 64));
    }
    static int set_split(GemmDesc& d, int ks) {
        const int kchunk = ((d.K + ks - 1) / ks + 15) / 16 * 16;
        d.kchunk = kchunk;
        d.ksplit = (d.K + kchunk - 1) / kchunk;
        return d.ksplit;
    }
    // panels bucketed by register class (0 = in place in global memory)
    void add_panel(std::vector<std::vector<PanelDesc>>& byc, std::vector<int>& maxh, const PanelDesc& pd) const {
        int cls = panel_rows_class(pd.h);
        if (cls > 0 && panel_lds_bytes(true, pd.h) > lds_limit) cls = 0;
        int bucket = 0;
        for (int i = 0; cls > 0 && i < PANEL_NCLASS; ++i)
            if (PANEL_CLASSES[i] == cls) bucket = i + 1;
        byc[bucket].push_back(pd);
        maxh[bucket] = std::max(maxh[bucket], pd.h);
    }
    void panel_launches(Seq& st, std::vector<std::vector<PanelDesc>>& byc, const std::vector<int>& maxh) {
        for (int b = 0; b <= PANEL_NCLASS; ++b) {
            if (byc[b].empty()) continue;
            std::vector<int> ones(byc[b].size(), 1);
            Launch L = make_items(K_PANEL, byc[b], ones);
            L.mode = b == 0 ? 0 : PANEL_CLASSES[b - 1];
            L.max_h = maxh[b];
            L.ntiles = (int)byc[b].size();
            for (const auto& pd : byc[b]) {
                L.flops += householder_flops(pd.h, pd.nb);
                L.bytes += 4.0 * (double)pd.h * pd.nb * 3;   // read the panel, write V and Y
            }
            st.push_back(L);
        }
    }
    // Algorithmic flops (the standard Householder counts; what the kernels add on top, the
    // triangular factor T and its products, is not counted):
    //   factorization of an h x nb panel                      2 h nb^2 - 2 nb^3 / 3
    //   nb reflectors of length h applied to c columns         4 h nb c - 2 nb^2 c
    // Summed over the panels of a p x p matrix: (4/3) p^3 for the factorization and, with Q
    // formed by applying each panel to the h x h part of Q it reaches (c = h), another
    // (4/3) p^3 for Q.
    static double householder_flops(int h, int nb) {
        return 2.0 * h * nb * nb - 2.0 * nb * nb * nb / 3.0;
    }
    static double reflector_apply_flops(int h, int nb, int c) {
        return 4.0 * h * nb * c - 2.0 * (double)nb * nb * c;
    }
    static Launch sync_op(Kind k, int strm, int ev) {
        Launch L;
        L.kind = k;
        L.strm = strm;
        L.ev = ev;
        return L;
    }
    static void on_stream(Seq& seq, int strm) {
        for (auto& L : seq) L.strm = strm;
    }

    void build_qr_blocked() {
        // Householder QR of P, blocked twice (or once, when the outer width is 32).
        // Panels of 32 columns are factored one workgroup each; the panel's reflectors
        // are applied at once (compact WY) only to the rest of its outer block, and each panel's Y = V T is folded into
        // the outer block's Y (Y_b <- Y_b - Y_a (V_a^T Y_b), which is V T of the product
        // of all the block's reflectors).  After an outer block's last panel its
        // reflectors update the trailing columns (A <- A - V (Y^T A)) as products of depth
        // `outer`.  Q = H_0 H_1 ... is accumulated backward once every block is factored:
        // starting from I, block b updates only Q[C0:, C0:] (Q_s <- Q_s - Y (V^T Q_s)), which
        // costs 4 w h^2 flops per block instead of the 4 w h p of forward accumulation.
        // The columns of Q are flipped to diag(R) >= 0 at the end.
        qr_steps.assign(max_panels, Seq{});
        qr_join.clear();
        // Two groups of sides (alternate blocks) run their factorizations on two streams:
        // a panel launch takes one CU per side and leaves the rest of the GPU idle for its
        // whole chain of reflector steps, which the other group's matrix products fill.
        // The sides share no buffer; both groups join before Q is accumulated.
        const int ngroup = qr_split && max_panels > 0 && full.size() > 2 ? 2 : 1;
        std::vector<std::vector<std::reference_wrapper<Side>>> groups(ngroup);
        for (size_t i = 0; i < full.size(); ++i) groups[ngroup == 2 ? (i / 2) % 2 : 0].push_back(full[i]);
        if (ngroup == 2) {
            n_sync = 2;
            qr_steps[0].push_back(sync_op(K_RECORD, 0, 0));
            qr_steps[0].push_back(sync_op(K_WAIT, 1, 0));
        }
        for (int sidx = 0; sidx < max_panels; ++sidx)
        for (int grp = 0; grp < ngroup; ++grp) {
            const auto& gsides = groups[grp];
            // panels bucketed by register class (0 = in place in global memory)
            std::vector<std::vector<PanelDesc>> byc(PANEL_NCLASS + 1);
            std::vector<int> maxh(PANEL_NCLASS + 1, 0);
            std::vector<GemmItem> in1, in2, out1, out2;
            // split-K factors: chosen per launch so that a batch too small to fill the
            // GPU still spreads its long-K (K = panel height) products
            long tin = 0, tout = 0;
            int kin = 1 << 30, kout = 1 << 30;
            for (Side& S : gsides) {
                const int p = S.p, c0 = sidx * kPanel;
                if (c0 >= p) continue;
                const int C0 = c0 / outer * outer, wb = std::min(outer, p - C0);
                const int nbw = std::min(kPanel, p - c0), i = (c0 - C0) / kPanel;
                const int ninner = C0 + wb - c0 - nbw;
                tin += tiles64(nbw, ninner) + tiles64((long)i * kPanel, nbw);
                kin = std::min(kin, p - c0);
                if (ninner == 0) {
                    tout += tiles64(wb, p - C0 - wb);
                    kout = std::min(kout, p - C0);
                }
            }
            const int ks_in = split_for(tin, kin), ks_out = split_for(tout, kout);
            for (Side& S : gsides) {
                const int p = S.p;
                const int c0 = sidx * kPanel;
                if (c0 >= p) continue;
                const int C0 = c0 / outer * outer;
                const int wb = std::min(outer, p - C0);
                const int ho = p - C0;                       // rows of the outer block
                const int nbw = std::min(kPanel, p - c0);
                const int h = p - c0;
                const int i = (c0 - C0) / kPanel;            // panel index inside the block
                const int ninner = C0 + wb - c0 - nbw;       // block columns right of the panel
                const int ntr = p - C0 - wb;                 // columns right of the block
                float* Vo = wsf(S.Vb) + S.outer_rows[C0 / outer] * outer;
                float* Yo = wsf(S.Yb) + S.outer_rows[C0 / outer] * outer;
                float* Pm = wsf(S.Pm);
                float* Z = wsf(S.Z);
                float* Mb = wsf(S.Mb);
                const int64_t zslab = (int64_t)outer * p, mslab = (int64_t)outer * kPanel;
                PanelDesc pd;
                std::memset(&pd, 0, sizeof(pd));
                pd.A = Pm;
                pd.V = Vo + i * kPanel;
                pd.Y = Yo + i * kPanel;
                pd.rdiag = wsf(S.rdiag);
                pd.ld = p;
                pd.vld = outer;
                pd.c0 = c0;
                pd.h = h;
                pd.nb = nbw;
                pd.zrows = c0 - C0;
                add_panel(byc, maxh, pd);
                float* Vp = Vo + (int64_t)(c0 - C0) * outer + i * kPanel;   // panel's V, top row c0
                float* Yp = Yo + (int64_t)(c0 - C0) * outer + i * kPanel;
                if (ninner > 0) {   // the panel's reflectors on the rest of its outer block
                    float* Ab = Pm + (int64_t)c0 * p + c0 + nbw;
                    GemmDesc z = gd(Yp, outer, Ab, p, Z, p, nbw, ninner, h);
                    const int ns = set_split(z, ks_in);
                    z.dslab = zslab;
                    in1.push_back({z, true, false});
                    GemmDesc u = gd(Vp, outer, Z, p, Ab, p, h, ninner, nbw, -1.f, 1.f, Ab, p);
                    u.bnslab = ns; u.bslab = zslab;
                    in2.push_back({u, false, false});
                }
                if (i > 0) {        // fold this panel's Y into the block's
                    GemmDesc m = gd(Vo + (int64_t)(c0 - C0) * outer, outer, Yp, outer, Mb, kPanel,
                                    i * kPanel, nbw, h);
                    const int ns = set_split(m, ks_in);
                    m.dslab = mslab;
                    in1.push_back({m, true, false});
                    GemmDesc y = gd(Yo, outer, Mb, kPanel, Yo + i * kPanel, outer, ho, nbw, i * kPanel,
                                    -1.f, 1.f, Yo + i * kPanel, outer);
                    y.bnslab = ns; y.bslab = mslab;
                    in2.push_back({y, false, false});
                }
                if (ninner == 0 && ntr > 0) {  // last panel of the block: trailing columns
                    float* At = Pm + (int64_t)C0 * p + C0 + wb;
                    GemmDesc z = gd(Yo, outer, At, p, Z, p, wb, ntr, ho);
                    const int ns = set_split(z, ks_out);
                    z.dslab = zslab;
                    out1.push_back({z, true, false});
                    GemmDesc u = gd(Vo, outer, Z, p, At, p, ho, ntr, wb, -1.f, 1.f, At, p);
                    u.bnslab = ns; u.bslab = zslab;
                    out2.push_back({u, false, false});
                }
            }
            Seq gs;
            panel_launches(gs, byc, maxh);
            for (auto* items : {&in1, &in2, &out1, &out2}) {
                const int fam = (items == &out1 || items == &out2) ? FAM_GEMM_QR_TRAIL : FAM_GEMM_QR;
                Seq g = make_gemm(*items, fam, outer > kPanel);
                gs.insert(gs.end(), g.begin(), g.end());
            }
            on_stream(gs, grp);
            qr_steps[sidx].insert(qr_steps[sidx].end(), gs.begin(), gs.end());
        }
        if (ngroup == 2) {
            qr_steps.back().push_back(sync_op(K_RECORD, 1, 1));
            qr_steps.back().push_back(sync_op(K_WAIT, 0, 1));
        }
        // backward accumulation of Q (Q holds I): block b, last to first
        int max_outer = 0;
        for (Side& S : full) max_outer = std::max(max_outer, (S.p + outer - 1) / outer);
        for (int ob = max_outer - 1; ob >= 0; --ob) {
            std::vector<GemmItem> w1, w2;
            long tw = 0;
            int kw = 1 << 30;
            for (Side& S : full) {
                const int C0 = ob * outer;
                if (C0 >= S.p) continue;
                tw += tiles64(std::min(outer, S.p - C0), S.p - C0);
                kw = std::min(kw, S.p - C0);
            }
            const int ks_w = split_for(tw, kw);
            for (Side& S : full) {
                const int p = S.p, C0 = ob * outer;
                if (C0 >= p) continue;
                const int ho = p - C0, wb = std::min(outer, ho);
                const float* Vo = wsf(S.Vb) + S.outer_rows[ob] * outer;
                const float* Yo = wsf(S.Yb) + S.outer_rows[ob] * outer;
                float* Qs = wsf(S.Qm) + (int64_t)C0 * p + C0;   // Q[C0:, C0:]
                float* Wb = wsf(S.W);
                const int64_t wslab = (int64_t)outer * p;
                GemmDesc w = gd(Vo, outer, Qs, p, Wb, p, wb, ho, ho);   // W = V^T Q_s
                const int ns = set_split(w, ks_w);
                w.dslab = wslab;
                w1.push_back({w, true, false});
                GemmDesc q = gd(Yo, outer, Wb, p, Qs, p, ho, ho, wb, -1.f, 1.f, Qs, p);
                q.bnslab = ns; q.bslab = wslab;
                w2.push_back({q, false, false});
            }
            for (auto* items : {&w1, &w2}) {
                Seq g = make_gemm(*items, FAM_GEMM_QR_Q, outer > kPanel);
                qr_join.insert(qr_join.end(), g.begin(), g.end());
            }
        }
    }

    // Fused QR steps (panel-wide blocks, one launch per panel index k): the workgroup of
    // panel k first applies panel k-1's reflectors to its own 32 columns and then factors
    // them, while in the same launch other workgroups apply panel k-1's reflectors to the
    // trailing columns beyond panel k (32 at a time) and to Q (32 rows at a time).  A last
    // launch applies each side's final panel to Q.  The chain of launches is the chain of
    // panels; the matrix products ride along instead of following each panel.
    void build_qr_fused() {
        qr_steps.assign(max_panels + 1, Seq{});
        qr_join.clear();
        for (int k = 0; k <= max_panels; ++k) {
            std::vector<StepPanelDesc> pds;
            std::vector<SlabDesc> sds;
            int max_h = 0;
            double flops = 0, bytes = 0;
            for (Side& S : full) {
                const int p = S.p;
                float* Pm = wsf(S.Pm);
                float* Qm = wsf(S.Qm);
                auto vblock = [&](int panel) { return wsf(S.Vb) + S.outer_rows[panel] * kPanel; };
                auto tblock = [&](int panel) { return wsf(S.Tb) + (size_t)panel * kPanel * kPanel; };
                const int c0 = k * kPanel;
                if (c0 < p) {                                   // panel k
                    StepPanelDesc sp;
                    std::memset(&sp, 0, sizeof(sp));
                    PanelDesc& pd = sp.pd;
                    pd.A = Pm;
                    pd.V = vblock(k);
                    pd.Y = nullptr;
                    sp.T = tblock(k);
                    pd.rdiag = wsf(S.rdiag);
                    pd.ld = p;
                    pd.vld = kPanel;
                    pd.c0 = c0;
                    pd.h = p - c0;
                    pd.nb = std::min(kPanel, p - c0);
                    pd.zrows = 0;
                    if (k > 0) {
                        sp.Vp = vblock(k - 1);
                        sp.Tp = tblock(k - 1);
                        sp.nbp = kPanel;
                        sp.hp = pd.h + kPanel;
                        flops += reflector_apply_flops(sp.hp, kPanel, pd.nb);
                        bytes += 4.0 * (2.0 * sp.hp * kPanel + (double)kPanel * pd.nb + kPanel * kPanel);
                    }
                    pds.push_back(sp);
                    max_h = std::max(max_h, pd.h);
                    flops += householder_flops(pd.h, pd.nb);
                    bytes += 4.0 * (double)pd.h * pd.nb * 3;
                }
                const int r0 = (k - 1) * kPanel;
                if (k > 0 && r0 < p) {                          // panel k-1 on P and on Q
                    const int h = p - r0, nbk = std::min(kPanel, h);
                    const float* V = vblock(k - 1);
                    const float* T = tblock(k - 1);
                    for (int cs = c0 + kPanel; cs < p; cs += kPanel) {
                        SlabDesc sd;
                        std::memset(&sd, 0, sizeof(sd));
                        sd.M = Pm + (int64_t)r0 * p + cs;
                        sd.V = V; sd.T = T; sd.ld = p; sd.vld = kPanel;
                        sd.role = 0; sd.h = h; sd.count = std::min(kPanel, p - cs);
                        sds.push_back(sd);
                        flops += reflector_apply_flops(h, nbk, sd.count);
                        bytes += 4.0 * h * (2.0 * kPanel + 2.0 * sd.count);
                    }
                    for (int q0 = 0; q0 < p; q0 += kPanel) {
                        SlabDesc sd;
                        std::memset(&sd, 0, sizeof(sd));
                        sd.M = Qm + (int64_t)q0 * p + r0;
                        sd.V = V; sd.T = T; sd.ld = p; sd.vld = kPanel;
                        sd.role = 1; sd.h = h; sd.count = std::min(kPanel, p - q0);
                        // Q = I before the first block: the slabs take it as such and
                        // write all of Q (block 0 spans every column), so no fill runs
                        sd.ident = k == 1 ? 1 : 0;
                        sd.diag = q0 - r0;
                        sds.push_back(sd);
                        // Q is accumulated forward over all its rows here; the algorithmic
                        // count is that of applying the panel to the h x h part of Q it
                        // reaches (its share of the (4/3) p^3 of forming Q)
                        if (q0 == 0) flops += reflector_apply_flops(h, nbk, h);
                        bytes += 4.0 * h * (2.0 * kPanel + 2.0 * sd.count);
                    }
                }
            }
            if (pds.empty() && sds.empty()) continue;
            Launch L;
            L.kind = K_QRSTEP;
            L.fam = FAM_PANEL;
            L.mode = pds.empty() ? 2 : panel_rows_class(max_h);
            L.max_h = max_h;
            L.ndesc = (int)pds.size();
            L.ntiles = (int)(pds.size() + sds.size());
            L.desc_off = blob_put(pds.data(), pds.size() * sizeof(StepPanelDesc));
            L.prefix_off = blob_put(sds.data(), sds.size() * sizeof(SlabDesc));
            L.flops = flops;
            L.bytes = bytes;
            qr_steps[k].push_back(L);
        }
    }

    // Panel-wide reflector blocks with look-ahead.  The caller's stream runs the chain
    // of panels: panel k, then H_k applied to panel k+1's columns only.  The second
    // stream applies H_k to the columns beyond and accumulates Q; panel k+1's own
    // look-ahead update waits for that trailing update of k.  Event k of each kind is
    // recorded once per pass, before any wait on it is enqueued.
    void build_qr_lookahead() {
        qr_steps.assign(max_panels, Seq{});
        qr_join.clear();
        const int evA = 0, evR = max_panels, evEnd = 2 * max_panels;
        n_sync = 2 * max_panels + 1;
        for (int sidx = 0; sidx < max_panels; ++sidx) {
            std::vector<std::vector<PanelDesc>> byc(PANEL_NCLASS + 1);
            std::vector<int> maxh(PANEL_NCLASS + 1, 0);
            std::vector<GemmItem> la1, la2, r1, r2, q1, q2;
            long tla = 0, trest = 0;
            int kmin = 1 << 30;
            for (Side& S : full) {
                const int p = S.p, c0 = sidx * kPanel;
                if (c0 >= p) continue;
                const int nbw = std::min(kPanel, p - c0);
                const int nxt = std::min(kPanel, p - c0 - nbw);
                tla += tiles64(nbw, nxt);
                trest += tiles64(nbw, p - c0 - nbw - nxt) + tiles64(p, nbw);
                kmin = std::min(kmin, p - c0);
            }
            const int ks_la = split_for(tla, kmin), ks_rest = split_for(trest, kmin);
            for (Side& S : full) {
                const int p = S.p;
                const int c0 = sidx * kPanel;
                if (c0 >= p) continue;
                const int nbw = std::min(kPanel, p - c0);
                const int h = p - c0;
                const int nxt = std::min(kPanel, p - c0 - nbw);     // look-ahead columns
                const int nrest = p - c0 - nbw - nxt;
                float* Vp = wsf(S.Vb) + S.outer_rows[sidx] * kPanel;
                float* Yp = wsf(S.Yb) + S.outer_rows[sidx] * kPanel;
                float* Pm = wsf(S.Pm);
                PanelDesc pd;
                std::memset(&pd, 0, sizeof(pd));
                pd.A = Pm; pd.V = Vp; pd.Y = Yp; pd.rdiag = wsf(S.rdiag);
                pd.ld = p; pd.vld = kPanel;
                pd.c0 = c0; pd.h = h; pd.nb = nbw; pd.zrows = 0;
                add_panel(byc, maxh, pd);
                if (nxt > 0) {
                    float* An = Pm + (int64_t)c0 * p + c0 + nbw;
                    float* Z2 = wsf(S.Z2);
                    GemmDesc z = gd(Yp, kPanel, An, p, Z2, kPanel, nbw, nxt, h);
                    const int ns = set_split(z, ks_la);
                    z.dslab = (int64_t)kPanel * kPanel;
                    la1.push_back({z, true, false});
                    GemmDesc u = gd(Vp, kPanel, Z2, kPanel, An, p, h, nxt, nbw, -1.f, 1.f, An, p);
                    u.bnslab = ns; u.bslab = (int64_t)kPanel * kPanel;
                    la2.push_back({u, false, false});
                }
                if (nrest > 0) {
                    float* At = Pm + (int64_t)c0 * p + c0 + nbw + nxt;
                    float* Z = wsf(S.Z);
                    GemmDesc z = gd(Yp, kPanel, At, p, Z, p, nbw, nrest, h);
                    const int ns = set_split(z, ks_rest);
                    z.dslab = (int64_t)kPanel * p;
                    r1.push_back({z, true, false});
                    GemmDesc u = gd(Vp, kPanel, Z, p, At, p, h, nrest, nbw, -1.f, 1.f, At, p);
                    u.bnslab = ns; u.bslab = (int64_t)kPanel * p;
                    r2.push_back({u, false, false});
                }
                float* Qs = wsf(S.Qm) + c0;
                float* Wb = wsf(S.W);
                GemmDesc w = gd(Qs, p, Yp, kPanel, Wb, kPanel, p, nbw, h);
                const int ns = set_split(w, ks_rest);
                w.dslab = (int64_t)p * kPanel;
                q1.push_back({w, false, false});
                GemmDesc q = gd(Wb, kPanel, Vp, kPanel, Qs, p, p, h, nbw, -1.f, 1.f, Qs, p);
                q.anslab = ns; q.aslab = (int64_t)p * kPanel;
                q2.push_back({q, false, true});
            }
            Seq& st = qr_steps[sidx];
            panel_launches(st, byc, maxh);
            if (sidx > 0) st.push_back(sync_op(K_WAIT, 0, evR + sidx - 1));
            for (auto* items : {&la1, &la2}) {
                Seq g = make_gemm(*items, FAM_GEMM_QR);
                st.insert(st.end(), g.begin(), g.end());
            }
            st.push_back(sync_op(K_RECORD, 0, evA + sidx));
            st.push_back(sync_op(K_WAIT, 1, evA + sidx));
            for (auto* items : {&r1, &r2}) {
                Seq g = make_gemm(*items, FAM_GEMM_QR);
                on_stream(g, 1);
                st.insert(st.end(), g.begin(), g.end());
            }
            st.push_back(sync_op(K_RECORD, 1, evR + sidx));
            for (auto* items : {&q1, &q2}) {
                Seq g = make_gemm(*items, FAM_GEMM_QR);
                on_stream(g, 1);
                st.insert(st.end(), g.begin(), g.end());
            }
        }
        qr_join.push_back(sync_op(K_RECORD, 1, evEnd));
        qr_join.push_back(sync_op(K_WAIT, 0, evEnd));
    }

    void build() {
        blob.clear();
        const float beta = cfg.beta;
        build_bjorck(true, deq_root, bj_root);
        if (fp64) build_fp64();
        else build_stats_fp32(beta);
        build_tail();
    }

    // The float32 statistics update: Bjorck, the statistic, the power step and the QR
    // schedule the batch calls for.
    void build_stats_fp32(float beta) {
        build_bjorck(false, deq_stats, bj_stats);
        // statistics: Lt = beta V diag(lam) V^T, then Lt += (1 - beta) G G^T (side R: G^T G)
        for (int var = 0; var < 2; ++var) {
            std::vector<GemmItem> xs, pw;
            for (Side& S : full) {
                const int p = S.p;
                const float* V = wsf(var == 0 ? S.Vs : S.Vr);
                GemmDesc d = gd(V, p, V, p, wsf(S.Lt), p, p, p, p, beta);
                d.kscale = stf(S.lam);
                d.flags |= GEMM_F_SYM;                   // V diag(lam) V^T
                xs.push_back({d, false, true});
                pw.push_back({gd(wsf(S.Lt), p, V, p, wsf(S.Pm), p, p, p, p), false, false});
            }
            stats_x[var] = make_gemm(xs, FAM_GEMM_STATS);
            power_first[var] = make_gemm(pw, FAM_GEMM_POWER);
        }
        {
            std::vector<GemmItem> gs, pn;
            for (int b = 0; b < nb; ++b) {
                for (int s = 0; s < 2; ++s) {
                    Side& S = sides[2 * b + s];
                    if (S.diag) continue;
                    const int p = S.p, q = S.q;
                    GemmDesc d = gd(nullptr, 0, nullptr, 0, wsf(S.Lt), p, p, p, q, 1.f - beta, 1.f,
                                    wsf(S.Lt), p);
                    d.a_io = d.b_io = b;
                    d.flags |= GEMM_F_SYM;               // G G^T (G^T G), added to a symmetric Lt
                    gs.push_back({d, s == 1, s == 0});
                    pn.push_back({gd(wsf(S.Lt), p, wsf(S.Qm), p, wsf(S.Pm), p, p, p, p), false, false});
                }
            }
            stats_g = make_gemm(gs, FAM_GEMM_STATS);
            power_next = make_gemm(pn, FAM_GEMM_POWER);
            // folded form: Lt = (1 - beta) G G^T in the Gram launch, then += beta V diag(lam) V^T
            // (taken when the Gram launch leaves the GPU's workgroup slots idle; a full
            // one would gain only a launch and lose the single-transpose kernel)
            bj_stats_fold.clear();
            stats_x_fold.clear();
            long gram_tiles = 0;   // 128 x 128 tiles of the Gram products
            for (Side& S : full) {
                const long t = (S.p + 127) / 128;
                gram_tiles += t * (t + 1) / 2;
            }
            if (cfg.bjorck_iters > 0 && gram_tiles < 512) {
                for (auto& it : gs) {
                    it.d.beta = 0.f;
                    it.d.C = nullptr;
                }
                Seq unused;
                build_bjorck(false, unused, bj_stats_fold, &gs);
                std::vector<GemmItem> xs;
                for (Side& S : full) {
                    const int p = S.p;
                    const float* V = wsf(S.Vs);
                    GemmDesc d = gd(V, p, V, p, wsf(S.Lt), p, p, p, p, beta, 1.f, wsf(S.Lt), p);
                    d.kscale = stf(S.lam);
                    d.flags |= GEMM_F_SYM;
                    xs.push_back({d, false, true});
                }
                stats_x_fold = make_gemm(xs, FAM_GEMM_STATS);
            }
        }

        {   // panel-wide blocks on one stream run as fused QR steps when every panel fits
            // the register-resident kernel (and the device's LDS)
            int pmax = 0;
            for (Side& S : full) pmax = std::max(pmax, S.p);
            fused = outer == kPanel && !lookahead && pmax <= PANEL_LDS_MAX_ROWS &&
                    qr_step_lds_bytes(pmax) <= lds_limit;
        }
        if (lookahead) build_qr_lookahead();
        else if (fused) build_qr_fused();
        else build_qr_blocked();
    }

    // Everything after the statistics and QR: the Rayleigh step, requantization, root
    // refresh, initial state, precondition and the diagonal sides.
    void build_tail() {
        {
            std::vector<VecDesc> qi, rr, rt;
            std::vector<int> tqi, trr, trt;
            std::vector<GemmItem> yg;
            std::vector<CodecDesc> qd, cp;
            std::vector<int> tq, tcp;
            std::vector<InitDesc> in;
            std::vector<int> tin;
            double qbytes = 0;
            for (auto& S : sides) {
                const int p = S.p;
                VecDesc v;
                if (S.diag) {   // the diagonal statistic: its root scaling and initial state only
                    std::memset(&v, 0, sizeof(v));
                    v.a = stf(S.lam); v.out = stf(S.d); v.p = p;
                    rt.push_back(v);
                    trt.push_back((p + 255) / 256);
                    InitDesc id;
                    std::memset(&id, 0, sizeof(id));
                    id.lam = stf(S.lam); id.d = stf(S.d); id.p = p; id.kind = INIT_DIAG;
                    in.push_back(id);
                    tin.push_back((p + 255) / 256);
                    continue;
                }
                std::memset(&v, 0, sizeof(v));
                v.out = wsf(S.Qm); v.aux = wsf(S.rdiag); v.ld = p; v.p = p;
                qi.push_back(v);
                tqi.push_back(fill_tiles(p));
                // Rayleigh: partial column sums of Q .* (L~ Q) per row tile into Wg
                GemmDesc d = gd(wsf(S.Lt), p, wsf(S.Qm), p, wsf(S.Wg), p, p, p, p, 1.f, 0.f, wsf(S.Qm), p);
                d.flags = GEMM_F_COLDOT;
                yg.push_back({d, false, false});
                std::memset(&v, 0, sizeof(v));
                v.a = stf(S.lam); v.out = stf(S.d); v.p = p;
                rt.push_back(v);
                trt.push_back((p + 255) / 256);
                CodecDesc c;
                std::memset(&c, 0, sizeof(c));
                c.x_in = wsf(S.Qm); c.codes_out = stp<uint8_t>(S.codes); c.scales_out = stf(S.scales);
                c.n = (int64_t)p * p;
                qd.push_back(c);
                tq.push_back((int)quant_tiles(c.n));
                qbytes += (double)p * p * (4.0 + 0.5 + 4.0 / 64);
                std::memset(&c, 0, sizeof(c));
                c.codes_in = stp<uint8_t>(S.codes); c.scales_in = stf(S.scales);
                c.codes_out = stp<uint8_t>(S.rcodes); c.scales_out = stf(S.rscales);
                c.n = (int64_t)p * p;
                cp.push_back(c);
                tcp.push_back((int)((S.nqb * 32 + COPY_TILE - 1) / COPY_TILE));
                InitDesc id;
                std::memset(&id, 0, sizeof(id));
                id.codes = stp<uint8_t>(S.codes); id.scales = stf(S.scales); id.lam = stf(S.lam);
                id.rcodes = stp<uint8_t>(S.rcodes); id.rscales = stf(S.rscales); id.d = stf(S.d);
                id.p = p;
                in.push_back(id);
                tin.push_back((int)((std::max<int64_t>(S.nqb, p) + 255) / 256));
            }
            qinit = {make_items(K_IDENTITY, qi, tqi)};
            qinit_signed = {make_items(K_IDENTITY, qi, tqi)};
            qinit_signed[0].mode = 1;
            sign = {make_items(K_SIGN, qi, tqi)};
            ray_gemm = make_gemm(yg, FAM_GEMM_RAYLEIGH);
            int bm = 32, bn = 128;
            gemm_tile_dims(ray_gemm.empty() ? GEMM_32x128 : ray_gemm[0].cfg, &bm, &bn);
            for (Side& S : full) {
                VecDesc v;
                std::memset(&v, 0, sizeof(v));
                v.a = wsf(S.Wg); v.out = stf(S.lam); v.ld = S.p; v.p = S.p; v.rows = (S.p + bm - 1) / bm;
                rr.push_back(v);
                trr.push_back((S.p + 255) / 256);
            }
            rayleigh = {make_items(K_RAYLEIGH, rr, trr)};
            if (fp64) {   // the float64 update has its own (s64_*): these float32 ones never run
                qinit.clear(); qinit_signed.clear(); sign.clear(); ray_gemm.clear(); rayleigh.clear();
            }
            root_d = {make_items(K_ROOT, rt, trt)};
            if (fp32_state) {
                std::vector<VecDesc> qv, rv;
                std::vector<int> qt;
                for (Side& S : full) {
                    const int64_t n = (int64_t)S.p * S.p;
                    qv.push_back(copyf_desc(wsf(S.Qm), stf(S.codes), n));
                    rv.push_back(copyf_desc(stf(S.codes), stf(S.rcodes), n));
                    qt.push_back(copyf_tiles(n));
                }
                Launch Lq = make_items(K_COPYF, qv, qt);
                Lq.fam = FAM_QUANT;
                Lq.mode = 1;   // check finiteness
                for (Side& S : full) Lq.bytes += (double)S.p * S.p * 8.0;
                quant = {Lq};
                root_copy = {make_items(K_COPYF, rv, qt)};
                for (auto& d : in)
                    if (d.kind == INIT_4BIT) d.kind = INIT_FP32;
            } else {
                Launch Lq = make_items(K_QUANT, qd, tq);
                Lq.bytes = qbytes;
                quant = {Lq};
                root_copy = {make_items(K_COPY, cp, tcp)};
            }
            init_seq = {make_items(K_INIT, in, tin)};
        }
        // precondition: X1 = diag(d_L) V_L^T G; X2 = X1 V_R diag(d_R); X1 = V_L X2; P = X1 V_R^T
        {
            std::vector<GemmItem> p1, p2, p3, p4;
            for (int b = 0; b < nb; ++b) {
                const Side& L = sides[2 * b];
                const Side& R = sides[2 * b + 1];
                const int m = shapes[b].m, n = shapes[b].n;
                if (L.diag && R.diag) continue;       // diag(d_L) G diag(d_R): diag_pre
                if (R.diag) {                         // X1 = diag(d_L) V_L^T G; P = V_L X1 diag(d_R)
                    GemmDesc d1 = gd(wsf(L.Vr), m, nullptr, 0, wsf(X1[b]), n, m, n, m);
                    d1.b_io = b;
                    d1.rscale = stf(L.d);
                    p1.push_back({d1, true, false});
                    GemmDesc d2 = gd(wsf(L.Vr), m, wsf(X1[b]), n, nullptr, 0, m, n, m);
                    d2.d_io = b;
                    d2.cscale = stf(R.d);
                    p2.push_back({d2, false, false});
                    continue;
                }
                if (L.diag) {                         // X1 = G V_R diag(d_R); P = diag(d_L) X1 V_R^T
                    GemmDesc d1 = gd(nullptr, 0, wsf(R.Vr), n, wsf(X1[b]), n, m, n, n);
                    d1.a_io = b;
                    d1.cscale = stf(R.d);
                    p1.push_back({d1, false, false});
                    GemmDesc d2 = gd(wsf(X1[b]), n, wsf(R.Vr), n, nullptr, 0, m, n, n);
                    d2.d_io = b;
                    d2.rscale = stf(L.d);
                    p2.push_back({d2, false, true});
                    continue;
                }
                GemmDesc d1 = gd(wsf(L.Vr), m, nullptr, 0, wsf(X1[b]), n, m, n, m);
                d1.b_io = b;
                d1.rscale = stf(L.d);
                p1.push_back({d1, true, false});
                GemmDesc d2 = gd(wsf(X1[b]), n, wsf(R.Vr), n, wsf(X2[b]), n, m, n, n);
                d2.cscale = stf(R.d);
                p2.push_back({d2, false, false});
                p3.push_back({gd(wsf(L.Vr), m, wsf(X2[b]), n, wsf(X1[b]), n, m, n, m), false, false});
                GemmDesc d4 = gd(wsf(X1[b]), n, wsf(R.Vr), n, nullptr, 0, m, n, n);
                d4.d_io = b;
                p4.push_back({d4, false, true});
            }
            pre[0] = make_gemm(p1, FAM_GEMM_PRECOND);
            pre[1] = make_gemm(p2, FAM_GEMM_PRECOND);
            pre[2] = make_gemm(p3, FAM_GEMM_PRECOND);
            pre[3] = make_gemm(p4, FAM_GEMM_PRECOND);
        }
        // with ROOT_CACHE the root matrices V^r diag(d) V^r^T are formed once per root refresh
        // and precondition is X1 = Rt_L G, P = X1 Rt_R (same product, other association)
        {
            std::vector<GemmItem> rm, q1, q2;
            for (Side& S : full) {
                GemmDesc d = gd(wsf(S.Vr), S.p, wsf(S.Vr), S.p, wsf(S.Rt), S.p, S.p, S.p, S.p);
                d.kscale = stf(S.d);
                d.flags |= GEMM_F_SYM;                   // V diag(d) V^T
                rm.push_back({d, false, true});
            }
            for (int b = 0; b < nb; ++b) {
                const Side& L = sides[2 * b];
                const Side& R = sides[2 * b + 1];
                const int m = shapes[b].m, n = shapes[b].n;
                if (L.diag && R.diag) continue;       // diag_pre
                if (R.diag) {                         // P = Rt_L G diag(d_R)
                    GemmDesc d1 = gd(wsf(L.Rt), m, nullptr, 0, nullptr, 0, m, n, m);
                    d1.b_io = b;
                    d1.d_io = b;
                    d1.cscale = stf(R.d);
                    q1.push_back({d1, false, false});
                    continue;
                }
                if (L.diag) {                         // P = diag(d_L) G Rt_R
                    GemmDesc d1 = gd(nullptr, 0, wsf(R.Rt), n, nullptr, 0, m, n, n);
                    d1.a_io = b;
                    d1.d_io = b;
                    d1.rscale = stf(L.d);
                    q1.push_back({d1, false, false});
                    continue;
                }
                GemmDesc d1 = gd(wsf(L.Rt), m, nullptr, 0, wsf(X1[b]), n, m, n, m);
                d1.b_io = b;
                q1.push_back({d1, false, false});
                GemmDesc d2 = gd(wsf(X1[b]), n, wsf(R.Rt), n, nullptr, 0, m, n, n);
                d2.d_io = b;
                q2.push_back({d2, false, false});
            }
            root_mat = make_gemm(rm, FAM_GEMM_PRECOND);
            // the copy beside the QR chain takes each launch's products on 128 x 128 tiles
            // on the same kind of matrix core: both forms sum each output over K in the
            // same order (one group of waves per tile, the same steps per 16 k, whatever
            // the tile), so P is bit-identical whichever runs
            const std::vector<GemmItem>* qs[2] = {&q1, &q2};
            for (int i = 0; i < 2; ++i) {
                std::vector<std::vector<GemmItem>> groups;
                pre_cached[i] = make_gemm(*qs[i], FAM_GEMM_PRECOND, false, true, &groups);
                pre_side[i].clear();
                for (size_t g = 0; g < groups.size(); ++g) {
                    Seq sq = gemm_launch(groups[g], FAM_GEMM_PRECOND, GEMM_128x128, gemm_cfg_x3(pre_cached[i][g].cfg));
                    pre_side[i].insert(pre_side[i].end(), sq.begin(), sq.end());
                }
            }
            for (auto& sq : pre_cached)
                for (auto& L : sq)
                    if (L.cfg == GEMM_64x64_K2) L.cfg = GEMM_64x64;
        }
        build_diag();
    }

    // Diagonal sides: the partial sums of G^2 and their EMA into the statistic (update),
    // and P = diag(d_L) G diag(d_R) for blocks whose two sides are diagonal (precondition).
    void build_diag() {
        diag_stats.clear();
        diag_pre.clear();
        std::vector<DiagDesc> parts, scale;
        std::vector<int> tparts, tscale;
        std::vector<VecDesc> ema;
        std::vector<int> tema;
        double pbytes = 0, ebytes = 0, sbytes = 0;
        for (int b = 0; b < nb; ++b) {
            const Side& L = sides[2 * b];
            const Side& R = sides[2 * b + 1];
            if (!L.diag && !R.diag) continue;
            const int m = shapes[b].m, n = shapes[b].n;
            const int tm = (m + DIAG_TR - 1) / DIAG_TR, tn = (n + DIAG_TC - 1) / DIAG_TC;
            DiagDesc d;
            std::memset(&d, 0, sizeof(d));
            d.rowpart = L.diag ? wsf(RP[b]) : nullptr;
            d.colpart = R.diag ? wsf(CP[b]) : nullptr;
            d.d_l = stf(L.d);
            d.d_r = stf(R.d);
            d.m = m; d.n = n; d.blk = b; d.tiles_n = tn;
            parts.push_back(d);
            tparts.push_back(tm * tn);
            pbytes += 4.0 * m * n + (L.diag ? 4.0 * tn * m : 0) + (R.diag ? 4.0 * tm * n : 0);
            for (int s = 0; s < 2; ++s) {
                const Side& S = sides[2 * b + s];
                if (!S.diag) continue;
                VecDesc v;
                std::memset(&v, 0, sizeof(v));
                v.a = wsf(s == 0 ? RP[b] : CP[b]);
                v.out = stf(S.lam);
                v.ld = S.p;
                v.p = S.p;
                v.rows = s == 0 ? tn : tm;
                ema.push_back(v);
                tema.push_back((S.p + 255) / 256);
                ebytes += 4.0 * S.p * (v.rows + 2);
            }
            if (L.diag && R.diag) {
                scale.push_back(d);
                tscale.push_back((m + diag_scale_rows(n) - 1) / diag_scale_rows(n));
                sbytes += 8.0 * m * n + 4.0 * (m + n);
            }
        }
        if (!parts.empty()) {
            Launch a = make_items(K_DIAG_PARTIALS, parts, tparts);
            a.bytes = pbytes;
            a.uses_io = true;
            Launch e = make_items(K_DIAG_EMA, ema, tema);
            e.bytes = ebytes;
            diag_stats = {a, e};
        }
        if (!scale.empty()) {
            Launch c = make_items(K_DIAG_SCALE, scale, tscale);
            c.bytes = sbytes;
            c.uses_io = true;
            diag_pre = {c};
        }
    }

    // ---- float64 statistics update (FP64_REFRESH) ------------------------------------
    struct G64Item {
        Gemm64Desc d;
        int mode;      // GEMM_F_TA | GEMM_F_TB
        bool f32in;    // float operands (the gradients, through the io table)
    };
    double* wsd(size_t off) const { return wsp<double>(off); }
    static Gemm64Desc g64(const void* A, int64_t lda, const void* B, int64_t ldb, double* D, int64_t ldd, int M,
                          int N, int K, double alpha = 1.0, double beta = 0.0, const double* C = nullptr,
                          int64_t ldc = 0) {
        Gemm64Desc d;
        std::memset(&d, 0, sizeof(d));
        d.A = A; d.B = B; d.C = C; d.D = D;
        d.lda = lda; d.ldb = ldb; d.ldc = ldc ? ldc : ldd; d.ldd = ldd;
        d.M = M; d.N = N; d.K = K;
        d.alpha = alpha; d.beta = beta;
        d.a_io = d.b_io = -1;
        return d;
    }
    // one launch per (transpose mode, operand type) present among the items
    Seq gemm64_seq(const std::vector<G64Item>& items, int fam) {
        Seq out;
        for (int f = 0; f < 2; ++f)
            for (int mode = 0; mode < 4; ++mode) {
                std::vector<Gemm64Desc> ds;
                std::vector<int> tiles;
                double flops = 0, bytes = 0;
                bool io_used = false;
                for (auto& it : items) {
                    if (it.mode != mode || (int)it.f32in != f || it.d.M <= 0 || it.d.N <= 0) continue;
                    Gemm64Desc d = it.d;
                    d.tiles_m = gemm64_tiles_m(d.M);
                    ds.push_back(d);
                    tiles.push_back(gemm64_tiles(d.M, d.N));
                    flops += 2.0 * d.M * d.N * d.K;
                    bytes += (f ? 4.0 : 8.0) * ((double)d.M * d.K + (double)d.K * d.N) +
                             8.0 * d.M * d.N * (d.beta != 0.0 ? 2 : 1);
                    io_used = io_used || d.a_io >= 0 || d.b_io >= 0;
                }
                if (ds.empty()) continue;
                Launch L = make_items(K_GEMM64, ds, tiles);
                L.fam = fam;
                L.mode = mode;
                L.f32in = f != 0;
                L.flops = flops;
                L.bytes = bytes;
                L.uses_io = io_used;
                out.push_back(L);
            }
        return out;
    }

    // U (dequantized, exact in float32) widened to float64; Bjorck, the statistic
    // beta V diag(lam) V^T + (1 - beta) G G^T, the power step, the Householder QR panel by
    // panel (each panel's reflectors on the columns right of it, then Q accumulated
    // backward from diag(sign(R_jj))), the Rayleigh quotients, all in float64; Q rounded
    // to float32 for the quantizer.  The same steps as the float32 update, in float64.
    void build_fp64() {
        const int k = cfg.bjorck_iters;
        const double beta = (double)cfg.beta;
        {   // U into Tmp (float32), then widened into V64a
            std::vector<CodecDesc> cds;
            std::vector<VecDesc> vd;
            std::vector<int> tiles, vt, ct;
            std::vector<Vec64Desc> cv;
            double bytes = 0;
            for (Side& S : full) {
                const int64_t n = (int64_t)S.p * S.p;
                if (fp32_state) {
                    vd.push_back(copyf_desc(stf(S.codes), wsf(S.Tmp), n));
                    vt.push_back(copyf_tiles(n));
                } else {
                    CodecDesc c;
                    std::memset(&c, 0, sizeof(c));
                    c.codes_in = stp<uint8_t>(S.codes);
                    c.scales_in = stf(S.scales);
                    c.x_out = wsf(S.Tmp);
                    c.n = n;
                    cds.push_back(c);
                    tiles.push_back((int)dequant_tiles(n));
                }
                bytes += (double)n * (fp32_state ? 8.0 : 4.0 + 0.5 + 4.0 / 64);
                Vec64Desc v;
                std::memset(&v, 0, sizeof(v));
                v.f32 = wsf(S.Tmp);
                v.out = wsd(S.V64a);
                v.p = S.p;
                cv.push_back(v);
                ct.push_back((int)((n + CVT_TILE - 1) / CVT_TILE));
            }
            Launch L = fp32_state ? make_items(K_COPYF, vd, vt) : make_items(K_DEQUANT, cds, tiles);
            L.fam = FAM_DEQUANT;
            L.bytes = bytes;
            Launch C = make_items(K_CVT, cv, ct);
            C.mode = 0;
            s64_pre = {L, C};
        }
        s64_bjorck.clear();
        for (int i = 0; i < k; ++i) {
            std::vector<G64Item> gram, upd;
            for (Side& S : full) {
                const int p = S.p;
                double* in = wsd(i % 2 == 0 ? S.V64a : S.V64b);
                double* out = wsd(i % 2 == 0 ? S.V64b : S.V64a);
                gram.push_back({g64(in, p, in, p, wsd(S.Wg64), p, p, p, p), GEMM_F_TA, false});
                upd.push_back({g64(in, p, wsd(S.Wg64), p, out, p, p, p, p, -0.5, 1.5, in, p), 0, false});
            }
            Seq sq = gemm64_seq(gram, FAM_GEMM64);
            Seq su = gemm64_seq(upd, FAM_GEMM64);
            sq.insert(sq.end(), su.begin(), su.end());
            s64_bjorck.push_back(sq);
        }
        auto vfin = [&](const Side& S) { return wsd(k % 2 == 0 ? S.V64a : S.V64b); };
        {   // the statistic, then the first and the later power steps
            std::vector<G64Item> xs, gs, pf, pn;
            for (Side& S : full) {
                const int p = S.p;
                Gemm64Desc d = g64(vfin(S), p, vfin(S), p, wsd(S.Lt64), p, p, p, p, beta);
                d.kscale = stf(S.lam);                    // V diag(lam) V^T
                xs.push_back({d, GEMM_F_TB, false});
                pf.push_back({g64(wsd(S.Lt64), p, vfin(S), p, wsd(S.P64), p, p, p, p), 0, false});
                pn.push_back({g64(wsd(S.Lt64), p, wsd(S.Q64), p, wsd(S.P64), p, p, p, p), 0, false});
            }
            for (int b = 0; b < nb; ++b)
                for (int s = 0; s < 2; ++s) {
                    Side& S = sides[2 * b + s];
                    if (S.diag) continue;
                    const int p = S.p, q = S.q;
                    Gemm64Desc d = g64(nullptr, 0, nullptr, 0, wsd(S.Lt64), p, p, p, q, 1.0 - beta, 1.0,
                                       wsd(S.Lt64), p);
                    d.a_io = d.b_io = b;   // G G^T (side R: G^T G), float gradients
                    gs.push_back({d, s == 0 ? GEMM_F_TB : GEMM_F_TA, true});
                }
            s64_stats = gemm64_seq(xs, FAM_GEMM64);
            Seq g = gemm64_seq(gs, FAM_GEMM64);
            s64_stats.insert(s64_stats.end(), g.begin(), g.end());
            s64_power_first = gemm64_seq(pf, FAM_GEMM64);
            s64_power_next = gemm64_seq(pn, FAM_GEMM64);
        }
        // QR of P64, panel by panel
        s64_qr.assign(max_panels, Seq{});
        s64_qacc.assign(max_panels, Seq{});
        for (int kp = 0; kp < max_panels; ++kp) {
            std::vector<Panel64Desc> pds;
            std::vector<int> ones;
            std::vector<G64Item> z1, z2, w1, w2;
            double pflops = 0;
            for (Side& S : full) {
                const int p = S.p, c0 = kp * kPanel;
                if (c0 >= p) continue;
                const int h = p - c0, nbw = std::min(kPanel, h), ntr = p - c0 - nbw;
                double* Vp = wsd(S.Vb64) + S.outer_rows[kp] * kPanel;
                double* Yp = wsd(S.Yb64) + S.outer_rows[kp] * kPanel;
                Panel64Desc pd;
                std::memset(&pd, 0, sizeof(pd));
                pd.A = wsd(S.P64); pd.V = Vp; pd.Y = Yp; pd.rdiag = wsd(S.rd64);
                pd.ld = p; pd.vld = kPanel; pd.c0 = c0; pd.h = h; pd.nb = nbw;
                pds.push_back(pd);
                ones.push_back(1);
                pflops += householder_flops(h, nbw);
                if (ntr > 0) {   // the panel's reflectors on the columns right of it: A -= V (Y^T A)
                    double* At = wsd(S.P64) + (int64_t)c0 * p + c0 + nbw;
                    z1.push_back({g64(Yp, kPanel, At, p, wsd(S.Z64), p, nbw, ntr, h), GEMM_F_TA, false});
                    z2.push_back({g64(Vp, kPanel, wsd(S.Z64), p, At, p, h, ntr, nbw, -1.0, 1.0, At, p), 0, false});
                }
                // Q accumulated backward: Q[c0:, c0:] -= Y (V^T Q[c0:, c0:])
                double* Qs = wsd(S.Q64) + (int64_t)c0 * p + c0;
                w1.push_back({g64(Vp, kPanel, Qs, p, wsd(S.W64), p, nbw, h, h), GEMM_F_TA, false});
                w2.push_back({g64(Yp, kPanel, wsd(S.W64), p, Qs, p, h, h, nbw, -1.0, 1.0, Qs, p), 0, false});
            }
            Launch P = make_items(K_PANEL64, pds, ones);
            P.fam = FAM_PANEL;
            P.flops = pflops;
            for (auto& pd : pds) P.bytes += 8.0 * (double)pd.h * pd.nb * 3;
            Seq& st = s64_qr[kp];
            st = {P};
            for (auto* items : {&z1, &z2}) {
                Seq g = gemm64_seq(*items, FAM_GEMM64);
                st.insert(st.end(), g.begin(), g.end());
            }
            Seq& qa = s64_qacc[max_panels - 1 - kp];   // run last panel first
            for (auto* items : {&w1, &w2}) {
                Seq g = gemm64_seq(*items, FAM_GEMM64);
                qa.insert(qa.end(), g.begin(), g.end());
            }
        }
        {   // Q = diag(sign(R_jj)) before the backward accumulation; Rayleigh; Q to float32
            std::vector<Vec64Desc> qi, cd, cq;
            std::vector<int> tqi, tcd, tcq;
            std::vector<G64Item> ray;
            for (Side& S : full) {
                const int p = S.p;
                Vec64Desc v;
                std::memset(&v, 0, sizeof(v));
                v.a = wsd(S.rd64); v.out = wsd(S.Q64); v.p = p;
                qi.push_back(v);
                tqi.push_back(p);
                ray.push_back({g64(wsd(S.Lt64), p, wsd(S.Q64), p, wsd(S.Wg64), p, p, p, p), 0, false});
                std::memset(&v, 0, sizeof(v));
                v.a = wsd(S.Q64); v.b = wsd(S.Wg64); v.f32 = stf(S.lam); v.p = p;
                cd.push_back(v);
                tcd.push_back((p + 255) / 256);
                std::memset(&v, 0, sizeof(v));
                v.a = wsd(S.Q64); v.f32 = wsf(S.Qm); v.p = p;
                cq.push_back(v);
                tcq.push_back((int)(((int64_t)p * p + CVT_TILE - 1) / CVT_TILE));
            }
            Launch I = make_items(K_IDENT64, qi, tqi);
            s64_qinit = {I};
            s64_post = gemm64_seq(ray, FAM_GEMM64);
            Launch D = make_items(K_COLDOT64, cd, tcd);
            D.fam = FAM_RAYLEIGH;
            Launch C = make_items(K_CVT, cq, tcq);
            C.mode = 1;
            s64_post.push_back(D);
            s64_post.push_back(C);
        }
    }

    // grafting epilogue: the same row tiles for both passes; bytes per element depend on
    // the mode (SGD: G, P read; Adam: also both moments read and written)
    void build_graft() {
        std::vector<GraftDesc> ds;
        std::vector<int> tiles;
        size_t t0 = 0;
        for (int b = 0; b < nb; ++b) {
            GraftDesc d;
            std::memset(&d, 0, sizeof(d));
            d.m = shapes[b].m;
            d.n = shapes[b].n;
            d.rows = graft_rows(d.n);
            d.blk = b;
            d.ntiles = (d.m + d.rows - 1) / d.rows;
            d.parts = wsf(parts_off) + 2 * t0;
            t0 += d.ntiles;
            ds.push_back(d);
            tiles.push_back(d.ntiles);
        }
        for (int mode = 0; mode < 2; ++mode) {
            Launch a = make_items(K_GRAFT_NORMS, ds, tiles);
            Launch u = make_items(K_GRAFT_APPLY, ds, tiles);
            for (auto& sh : shapes) {
                const double e = (double)sh.m * sh.n;
                a.bytes += e * (mode ? 24.0 : 8.0);
                u.bytes += e * 12.0;
            }
            graft_seq[mode] = {a, u};
        }
    }

    // ---- execution ------------------------------------------------------------
    hipError_t run(const Launch& L, hipStream_t caller) {
        const hipStream_t s = L.strm ? aux : caller;
        if (L.kind == K_RECORD) return hipEventRecord(sync_ev[L.ev], s);
        if (L.kind == K_WAIT) return hipStreamWaitEvent(s, sync_ev[L.ev], 0);
        const uint8_t* base = ws + desc_base;
        const int* prefix = reinterpret_cast<const int*>(base + L.prefix_off);
        const IoEntry* io = wsp<IoEntry>(io_off);
        uint32_t* flag = wsp<uint32_t>(flag_off);
        TimingRec rec{};
        if (timing) {
            rec.e0 = next_event();
            rec.e1 = next_event();
            launch_timing().start = rec.e0;
            launch_timing().stop = rec.e1;
        }
        hipError_t e = hipSuccess;
        const int fam = L.fam;
        switch (L.kind) {
            case K_GEMM:
                e = launch_gemm(L.cfg, L.mode, L.vec && (!L.uses_io || io_vec), L.slab, L.kscale,
                                reinterpret_cast<const GemmDesc*>(base + L.desc_off), prefix, L.ndesc, L.ntiles,
                                io, s);
                break;
            case K_DEQUANT:
                e = launch_dequant(codebook, reinterpret_cast<const CodecDesc*>(base + L.desc_off), prefix,
                                   L.ndesc, L.ntiles, s);
                break;
            case K_QUANT:
                e = launch_quant(codebook, reinterpret_cast<const CodecDesc*>(base + L.desc_off), prefix,
                                 L.ndesc, L.ntiles, flag, s);
                break;
            case K_COPY:
                e = launch_codec_copy(reinterpret_cast<const CodecDesc*>(base + L.desc_off), prefix,
                                      L.ndesc, L.ntiles, s);
                break;
            case K_PANEL:
                e = launch_panel(L.mode, reinterpret_cast<const PanelDesc*>(base + L.desc_off), L.ndesc,
                                 L.max_h, s);
                break;
            case K_QRSTEP:
                e = launch_qr_step(L.mode, reinterpret_cast<const StepPanelDesc*>(base + L.desc_off), L.ndesc,
                                   reinterpret_cast<const SlabDesc*>(base + L.prefix_off), L.ntiles - L.ndesc,
                                   L.max_h, s);
                break;
            case K_RAYLEIGH:
                e = launch_rayleigh_reduce(reinterpret_cast<const VecDesc*>(base + L.desc_off), prefix,
                                           L.ndesc, L.ntiles, flag, s);
                break;
            case K_ROOT:
                e = launch_root_scaling(reinterpret_cast<const VecDesc*>(base + L.desc_off), prefix,
                                        L.ndesc, L.ntiles, cfg.eps, flag, s);
                break;
            case K_IDENTITY:
                e = launch_identity_fill(reinterpret_cast<const VecDesc*>(base + L.desc_off), prefix,
                                         L.ndesc, L.ntiles, L.mode == 1, s);
                break;
            case K_SIGN:
                e = launch_sign_flip(reinterpret_cast<const VecDesc*>(base + L.desc_off), prefix, L.ndesc,
                                     L.ntiles, s);
                break;
            case K_INIT:
                e = launch_identity_state(reinterpret_cast<const InitDesc*>(base + L.desc_off), prefix,
                                          L.ndesc, L.ntiles, s);
                break;
            case K_NEWTON_NORM:
                e = launch_newton_norm(reinterpret_cast<const NewtonDesc*>(base + L.desc_off), prefix, L.ndesc,
                                       L.ntiles, newton_eps, s);
                break;
            case K_NEWTON_SCALE:
                e = launch_newton_scale(reinterpret_cast<const NewtonDesc*>(base + L.desc_off), L.ndesc, s);
                break;
            case K_NEWTON_ELEM:
                e = launch_newton_elem(reinterpret_cast<const NewtonDesc*>(base + L.desc_off), prefix, L.ndesc,
                                       L.ntiles, L.mode, newton_eps, s);
                break;
            case K_COPYF:
                e = launch_copyf(reinterpret_cast<const VecDesc*>(base + L.desc_off), prefix, L.ndesc, L.ntiles,
                                 L.mode ? flag : nullptr, s);
                break;
            case K_GRAFT_NORMS:
                e = launch_graft_norms(reinterpret_cast<const GraftDesc*>(base + L.desc_off), prefix, L.ndesc,
                                       L.ntiles, io, wsp<GraftIo>(gio_off), graft_prm, flag, s);
                break;
            case K_GRAFT_APPLY:
                e = launch_graft_apply(reinterpret_cast<const GraftDesc*>(base + L.desc_off), prefix, L.ndesc,
                                       L.ntiles, io, wsp<GraftIo>(gio_off), graft_prm, s);
                break;
            case K_GEMM64:
                e = launch_gemm64(L.mode, L.f32in, reinterpret_cast<const Gemm64Desc*>(base + L.desc_off), prefix,
                                  L.ndesc, L.ntiles, io, s);
                break;
            case K_PANEL64:
                e = launch_panel64(reinterpret_cast<const Panel64Desc*>(base + L.desc_off), L.ndesc, s);
                break;
            case K_COLDOT64:
                e = launch_coldot64(reinterpret_cast<const Vec64Desc*>(base + L.desc_off), prefix, L.ndesc, L.ntiles,
                                    flag, s);
                break;
            case K_IDENT64:
                e = launch_ident64(reinterpret_cast<const Vec64Desc*>(base + L.desc_off), prefix, L.ndesc, L.ntiles, s);
                break;
            case K_CVT:
                e = launch_cvt(reinterpret_cast<const Vec64Desc*>(base + L.desc_off), prefix, L.ndesc, L.ntiles,
                               L.mode, s);
                break;
            case K_DIAG_PARTIALS:
                e = launch_diag_partials(reinterpret_cast<const DiagDesc*>(base + L.desc_off), prefix, L.ndesc,
                                         L.ntiles, io, s);
                break;
            case K_DIAG_EMA:
                e = launch_diag_ema(reinterpret_cast<const VecDesc*>(base + L.desc_off), prefix, L.ndesc,
                                    L.ntiles, cfg.beta, flag, s);
                break;
            case K_DIAG_SCALE:
                e = launch_diag_scale(reinterpret_cast<const DiagDesc*>(base + L.desc_off), prefix, L.ndesc,
                                      L.ntiles, io, s);
                break;
            case K_RECORD:
            case K_WAIT:
                break;
        }
        if (timing) {
            // the launcher consumed the events only if it launched a kernel
            const bool launched = launch_timing().start == nullptr;
            launch_timing().start = launch_timing().stop = nullptr;
            if (launched) {
                rec.family = fam;
                rec.x3 = L.kind == K_GEMM && gemm_cfg_x3(L.cfg);
                rec.flops = L.flops;
                rec.bytes = L.bytes;
                recs.push_back(rec);
            }
        }
        return e;
    }

    hipError_t run(const Seq& seq, hipStream_t s) {
        for (const auto& L : seq) {
            hipError_t e = run(L, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }

    hipEvent_t next_event() {
        if (ev_used == ev_pool.size()) {
            hipEvent_t e;
            (void)hipEventCreate(&e);
            ev_pool.push_back(e);
        }
        return ev_pool[ev_used++];
    }

    hipError_t upload_io(const shampoo4_io* io, hipStream_t s) {
        io_vec = true;
        for (int b = 0; b < nb; ++b)
            io_vec = io_vec && (reinterpret_cast<uintptr_t>(io[b].G) & 15) == 0 && (io[b].ldg & 3) == 0 &&
                     (int64_t)(shapes[b].m - 1) * io[b].ldg + shapes[b].n < (int64_t(1) << 29);
        return upload_table(io, io_off, s);
    }

    // One per-call table (nb entries of 32 bytes) through a pinned staging slot.
    // A table equal to the one last uploaded to the same slot is not sent again (calls
    // on a context are ordered on one stream, so the device copy is already current).
    hipError_t upload_table(const void* table, size_t dev_off, hipStream_t s) {
        const size_t bytes = (size_t)nb * sizeof(IoEntry);
        std::vector<uint8_t>& last = dev_off == io_off ? last_io : last_gio;
        const uint8_t* src = static_cast<const uint8_t*>(table);
        if (last.size() == bytes && std::memcmp(last.data(), src, bytes) == 0) return hipSuccess;
        const int slot = ring_next;
        ring_next = (ring_next + 1) % kRing;
        if (ring_used[slot]) {
            hipError_t e = hipEventSynchronize(ring_ev[slot]);
            if (e != hipSuccess) return e;
        }
        uint8_t* dst = pinned + (size_t)slot * align_up(bytes);
        std::memcpy(dst, table, bytes);
        hipError_t e = hipMemcpyAsync(ws + dev_off, dst, bytes, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return e;
        ring_used[slot] = true;
        e = hipEventRecord(ring_ev[slot], s);
        if (e == hipSuccess) last.assign(src, src + bytes);
        return e;
    }

    // The kernels of one statistics update (everything after the io upload).
    // at_qr: called where the QR of the first power step begins (work forked from there
    // shares the GPU with the latency-bound panel chain rather than the products)
    hipError_t stats_body(bool reuse, hipStream_t s, const std::function<hipError_t()>* at_qr = nullptr) {
        const int var = reuse ? 1 : 0;
        hipError_t e = run(diag_stats, s);
        if (fp64) return stats_body_fp64(s, at_qr, e);
        const bool fold = !reuse && !bj_stats_fold.empty();
        if (!reuse && e == hipSuccess) {
            e = run(deq_stats, s);
            for (auto& it : (fold ? bj_stats_fold : bj_stats))
                if (e == hipSuccess) e = run(it, s);
        }
        if (fold) {
            if (e == hipSuccess) e = run(stats_x_fold, s);
        } else {
            if (e == hipSuccess) e = run(stats_x[var], s);
            if (e == hipSuccess) e = run(stats_g, s);
        }
        for (int it = 0; it < cfg.power_iters && e == hipSuccess; ++it) {
            e = run(it == 0 ? power_first[var] : power_next, s);
            if (e == hipSuccess && it == 0 && at_qr) e = (*at_qr)();
            // forward accumulation (fused and look-ahead schedules): Q = I (in the fused
            // steps the first Q slabs take it as given), reflectors, then the column signs;
            // backward (blocked): the factorization, then Q from the signs
            const bool backward_q = !fused && !lookahead;
            if (e == hipSuccess && !backward_q && !fused) e = run(qinit, s);
            for (size_t p = 0; p < qr_steps.size() && e == hipSuccess; ++p) e = run(qr_steps[p], s);
            if (e == hipSuccess && backward_q) e = run(qinit_signed, s);
            if (e == hipSuccess) e = run(qr_join, s);
            if (e == hipSuccess && !backward_q) e = run(sign, s);
        }
        if (e == hipSuccess) e = run(ray_gemm, s);
        if (e == hipSuccess) e = run(rayleigh, s);
        if (e == hipSuccess) e = run(quant, s);
        return e;
    }

    hipError_t stats_body_fp64(hipStream_t s, const std::function<hipError_t()>* at_qr, hipError_t e) {
        if (e == hipSuccess) e = run(s64_pre, s);
        for (auto& it : s64_bjorck)
            if (e == hipSuccess) e = run(it, s);
        if (e == hipSuccess) e = run(s64_stats, s);
        for (int it = 0; it < cfg.power_iters && e == hipSuccess; ++it) {
            e = run(it == 0 ? s64_power_first : s64_power_next, s);
            if (e == hipSuccess && it == 0 && at_qr) e = (*at_qr)();
            for (size_t p = 0; p < s64_qr.size() && e == hipSuccess; ++p) e = run(s64_qr[p], s);
            if (e == hipSuccess) e = run(s64_qinit, s);
            for (size_t p = 0; p < s64_qacc.size() && e == hipSuccess; ++p) e = run(s64_qacc[p], s);
        }
        if (e == hipSuccess) e = run(s64_post, s);
        if (e == hipSuccess) e = run(quant, s);
        return e;
    }

    // The statistics update after its io upload: graph replay or eager launches.
    // at_qr (optional): called where the QR begins (before the whole update when it is
    // replayed from a graph, after it when no power step runs)
    hipError_t submit_stats(hipStream_t s, const std::function<hipError_t()>* at_qr = nullptr) {
        // (the float64 update starts from the codes: the cached float32 root is not its V)
        const bool reuse = (cfg.flags & SHAMPOO4_FLAG_ROOT_CACHE) && root_v_valid && root_v_is_stats && !fp64;
        const int var = reuse ? 1 : 0, vi = io_vec ? 1 : 0;
        hipError_t e = hipSuccess;
        if (use_graphs && graph_ok && !timing) {
            if (!stats_graph[var][vi]) capture_stats(reuse);
            if (stats_graph[var][vi]) {
                if (at_qr) e = (*at_qr)();
                if (e == hipSuccess) e = hipGraphLaunch(stats_graph[var][vi], s);
            } else {
                e = stats_body(reuse, s, at_qr);
            }
        } else {
            e = stats_body(reuse, s, at_qr);
        }
        if (e == hipSuccess && at_qr && cfg.power_iters < 1) e = (*at_qr)();
        root_v_is_stats = false;
        return e;
    }

    // (each object is created once; a failed creation is retried on the next call)
    hipError_t ensure_pre_stream() {
        hipError_t e = hipSuccess;
        if (!pre_fork) e = hipEventCreateWithFlags(&pre_fork, hipEventDisableTiming);
        if (e == hipSuccess && !pre_join) e = hipEventCreateWithFlags(&pre_join, hipEventDisableTiming);
        if (e == hipSuccess && !pre_strm) e = hipStreamCreateWithFlags(&pre_strm, hipStreamNonBlocking);
        return e;
    }

    // Capture the statistics update once per variant (and gradient load width, io_vec
    // as set by the current call's upload) on the private stream; a failed capture turns
    // graphs off for the context (the calls then launch eagerly).
    void capture_stats(bool reuse) {
        const int var = reuse ? 1 : 0, vi = io_vec ? 1 : 0;
        if (!cap && hipStreamCreateWithFlags(&cap, hipStreamNonBlocking) != hipSuccess) {
            graph_ok = false;
            return;
        }
        if (hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal) != hipSuccess) {
            graph_ok = false;
            return;
        }
        const hipError_t e = stats_body(reuse, cap);
        hipGraph_t g = nullptr;
        const hipError_t e2 = hipStreamEndCapture(cap, &g);
        if (e != hipSuccess || e2 != hipSuccess || !g ||
            hipGraphInstantiate(&stats_graph[var][vi], g, nullptr, nullptr, 0) != hipSuccess) {
            stats_graph[var][vi] = nullptr;
            graph_ok = false;
        }
        if (g) (void)hipGraphDestroy(g);
        (void)hipGetLastError();
    }

    // Rectified root eigenvectors into Vr; with ROOT_CACHE also the root matrices.
    hipError_t root_eigenvectors(hipStream_t s) {
        hipError_t e = run(deq_root, s);
        for (auto& it : bj_root)
            if (e == hipSuccess) e = run(it, s);
        if (e == hipSuccess && (cfg.flags & SHAMPOO4_FLAG_ROOT_CACHE)) e = run(root_mat, s);
        return e;
    }
};

namespace {

shampoo4_status validate_cfg(const shampoo4_config* cfg) {
    if (!cfg) return SHAMPOO4_EINVAL;
    if (!(cfg->beta >= 0.f && cfg->beta <= 1.f)) return SHAMPOO4_EINVAL;
    if (!(cfg->eps >= 0.f) || !std::isfinite(cfg->eps)) return SHAMPOO4_EINVAL;
    if (cfg->qblock != 64) return SHAMPOO4_EINVAL;
    if (cfg->bjorck_iters < 0 || cfg->bjorck_iters > 16) return SHAMPOO4_EINVAL;
    if (cfg->power_iters < 1 || cfg->power_iters > 8) return SHAMPOO4_EINVAL;
    if (cfg->flags & ~(SHAMPOO4_FLAG_ROOT_CACHE | SHAMPOO4_FLAG_KEEP_STATE | SHAMPOO4_FLAG_QR_BLOCKED |
                       SHAMPOO4_FLAG_QR_LOOKAHEAD | SHAMPOO4_FLAG_FP32_STATE | SHAMPOO4_FLAG_GRAPHS |
                       SHAMPOO4_FLAG_DT_CODEBOOK | SHAMPOO4_FLAG_FP64_REFRESH | SHAMPOO4_FLAG_FP32_MFMA |
                       SHAMPOO4_FLAG_DEBUG))
        return SHAMPOO4_EINVAL;
    if ((cfg->flags & SHAMPOO4_FLAG_DT_CODEBOOK) && (cfg->flags & SHAMPOO4_FLAG_FP32_STATE))
        return SHAMPOO4_EINVAL;
    if ((cfg->flags & SHAMPOO4_FLAG_QR_BLOCKED) && (cfg->flags & SHAMPOO4_FLAG_QR_LOOKAHEAD))
        return SHAMPOO4_EINVAL;
    if ((cfg->flags & SHAMPOO4_FLAG_FP64_REFRESH) &&
        (cfg->flags & (SHAMPOO4_FLAG_QR_LOOKAHEAD | SHAMPOO4_FLAG_FP32_STATE)))
        return SHAMPOO4_EINVAL;
    return SHAMPOO4_OK;
}

shampoo4_status validate_shapes(int32_t nblocks, const shampoo4_shape* shapes, const uint8_t* diag_sides) {
    if (nblocks < 1 || nblocks > (1 << 20) || !shapes) return SHAMPOO4_EINVAL;
    for (int b = 0; b < nblocks; ++b) {
        const uint8_t dg = diag_sides ? diag_sides[b] : 0;
        if (dg & ~(SHAMPOO4_DIAG_L | SHAMPOO4_DIAG_R)) return SHAMPOO4_EINVAL;
        const int lim_m = (dg & SHAMPOO4_DIAG_L) ? kMaxDiagDim : kMaxDim;
        const int lim_n = (dg & SHAMPOO4_DIAG_R) ? kMaxDiagDim : kMaxDim;
        if (shapes[b].m < 1 || shapes[b].n < 1 || shapes[b].m > lim_m || shapes[b].n > lim_n)
            return SHAMPOO4_ESHAPE;
    }
    return SHAMPOO4_OK;
}

shampoo4_status validate_io(const shampoo4_ctx_s* c, const shampoo4_io* io, bool need_p) {
    if (!io) return SHAMPOO4_EINVAL;
    for (int b = 0; b < c->nb; ++b) {
        if (!io[b].G) return SHAMPOO4_EINVAL;
        if (io[b].ldg < c->shapes[b].n) return SHAMPOO4_ESHAPE;
        if (need_p) {
            if (!io[b].P) return SHAMPOO4_EINVAL;
            if (io[b].ldp < c->shapes[b].n) return SHAMPOO4_ESHAPE;
        }
    }
    return SHAMPOO4_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

std::unique_ptr<shampoo4_ctx_s> make_plan(const shampoo4_config* cfg, int32_t nblocks,
                                          const shampoo4_shape* shapes, const uint8_t* diag_sides) {
    auto c = std::make_unique<shampoo4_ctx_s>();
    c->cfg = *cfg;
    c->nb = nblocks;
    c->shapes.assign(shapes, shapes + nblocks);
    c->diag_bits.assign(nblocks, 0);
    if (diag_sides) c->diag_bits.assign(diag_sides, diag_sides + nblocks);
    c->lds_limit = 160 * 1024;
    c->layout();
    return c;
}

}  // namespace

extern "C" {

int32_t shampoo4_abi_version(void) { return SHAMPOO4_ABI_VERSION; }

const char* shampoo4_strerror(shampoo4_status s) {
    switch (s) {
        case SHAMPOO4_OK: return "ok";
        case SHAMPOO4_EINVAL: return "invalid argument";
        case SHAMPOO4_ESHAPE: return "invalid shape or leading dimension";
        case SHAMPOO4_EALIGN: return "buffer not 256-byte aligned";
        case SHAMPOO4_ESMALLBUF: return "buffer smaller than planned";
        case SHAMPOO4_EHIP: return "HIP runtime error";
        case SHAMPOO4_ENONFINITE: return "non-finite value seen on device";
    }
    return "unknown status";
}

shampoo4_status shampoo4_plan(const shampoo4_config* cfg, int32_t nblocks, const shampoo4_shape* shapes,
                              size_t* state_bytes, size_t* workspace_bytes) {
    return shampoo4_plan_ex(cfg, nblocks, shapes, nullptr, state_bytes, workspace_bytes);
}

shampoo4_status shampoo4_plan_ex(const shampoo4_config* cfg, int32_t nblocks, const shampoo4_shape* shapes,
                                 const uint8_t* diag_sides, size_t* state_bytes, size_t* workspace_bytes) {
    shampoo4_status st = validate_cfg(cfg);
    if (st != SHAMPOO4_OK) return st;
    if ((st = validate_shapes(nblocks, shapes, diag_sides)) != SHAMPOO4_OK) return st;
    if (!state_bytes || !workspace_bytes) return SHAMPOO4_EINVAL;
    auto c = make_plan(cfg, nblocks, shapes, diag_sides);
    c->build();   // null bases: only the sizes matter
    c->build_graft();
    *state_bytes = c->st_bytes;
    // slack: the panel launches are regrouped at init by the device's LDS limit
    *workspace_bytes = c->desc_base + align_up(c->blob.size()) + (size_t)c->max_panels * 8 * kAlign;
    return SHAMPOO4_OK;
}

shampoo4_status shampoo4_init(const shampoo4_config* cfg, int32_t nblocks, const shampoo4_shape* shapes,
                              void* state, size_t state_bytes, void* workspace, size_t workspace_bytes,
                              void* stream, shampoo4_ctx* out) {
    return shampoo4_init_ex(cfg, nblocks, shapes, nullptr, state, state_bytes, workspace, workspace_bytes, stream,
                            out);
}

shampoo4_status shampoo4_init_ex(const shampoo4_config* cfg, int32_t nblocks, const shampoo4_shape* shapes,
                                 const uint8_t* diag_sides, void* state, size_t state_bytes, void* workspace,
                                 size_t workspace_bytes, void* stream, shampoo4_ctx* out) {
    CallRange range_("shampoo4_init_ex");
    shampoo4_status st = validate_cfg(cfg);
    if (st != SHAMPOO4_OK) return st;
    if ((st = validate_shapes(nblocks, shapes, diag_sides)) != SHAMPOO4_OK) return st;
    if (!state || !workspace || !out) return SHAMPOO4_EINVAL;
    if ((reinterpret_cast<uintptr_t>(state) % kAlign) || (reinterpret_cast<uintptr_t>(workspace) % kAlign))
        return SHAMPOO4_EALIGN;
    auto c = make_plan(cfg, nblocks, shapes, diag_sides);
    {   // panel register classes are limited by what one workgroup may allocate in LDS
        int dev = 0, lds = 0;
        if (hipGetDevice(&dev) != hipSuccess) return SHAMPOO4_EHIP;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            return SHAMPOO4_EHIP;
        c->lds_limit = (size_t)lds;
    }
    c->st = static_cast<uint8_t*>(state);
    c->ws = static_cast<uint8_t*>(workspace);
    c->build();
    c->build_graft();
    if (c->bad_desc) return SHAMPOO4_EINVAL;   // debug: a descriptor reaches outside the buffers
    if (c->n_sync > 0) {   // second stream (default priority) and its synchronization events
        if (hipStreamCreateWithFlags(&c->aux, hipStreamNonBlocking) != hipSuccess) return SHAMPOO4_EHIP;
        c->sync_ev.assign(c->n_sync, nullptr);
        for (auto& ev : c->sync_ev)
            if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) return SHAMPOO4_EHIP;
    }
    const size_t need_ws = c->desc_base + align_up(c->blob.size());
    if (state_bytes < c->st_bytes || workspace_bytes < need_ws) return SHAMPOO4_ESMALLBUF;
    c->ws_bytes = need_ws;
    hipStream_t s = as_stream(stream);
    if (hipHostMalloc(reinterpret_cast<void**>(&c->pinned), kRing * align_up((size_t)nblocks * sizeof(IoEntry)),
                      hipHostMallocDefault) != hipSuccess)
        return SHAMPOO4_EHIP;
    for (auto& e : c->ring_ev)
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return SHAMPOO4_EHIP;
    if (hipMemcpyAsync(c->ws + c->desc_base, c->blob.data(), c->blob.size(), hipMemcpyHostToDevice, s) !=
        hipSuccess)
        return SHAMPOO4_EHIP;
    const uint32_t zero[4] = {0, 0, 0, 0};
    if (hipMemcpyAsync(c->ws + c->flag_off, zero, sizeof(zero), hipMemcpyHostToDevice, s) != hipSuccess)
        return SHAMPOO4_EHIP;
    if (!(cfg->flags & SHAMPOO4_FLAG_KEEP_STATE)) {
        if (c->run(c->init_seq, s) != hipSuccess) return SHAMPOO4_EHIP;
    }
    if (cfg->flags & SHAMPOO4_FLAG_ROOT_CACHE) {
        if (c->root_eigenvectors(s) != hipSuccess) return SHAMPOO4_EHIP;
        c->root_v_valid = true;
        c->root_v_is_stats = !(cfg->flags & SHAMPOO4_FLAG_KEEP_STATE);
    }
    if (hipStreamSynchronize(s) != hipSuccess) return SHAMPOO4_EHIP;
    *out = c.release();
    return SHAMPOO4_OK;
}

shampoo4_status shampoo4_update_stats(shampoo4_ctx c, const shampoo4_io* io, void* stream) {
    CallRange range_("shampoo4_update_stats");
    if (!c) return SHAMPOO4_EINVAL;
    shampoo4_status st = validate_io(c, io, false);
    if (st != SHAMPOO4_OK) return st;
    hipStream_t s = as_stream(stream);
    if (c->debug_fill(s) != hipSuccess) return SHAMPOO4_EHIP;
    if (c->upload_io(io, s) != hipSuccess) return SHAMPOO4_EHIP;
    return c->submit_stats(s) == hipSuccess ? SHAMPOO4_OK : SHAMPOO4_EHIP;
}

shampoo4_status shampoo4_refresh_root(shampoo4_ctx c, void* stream) {
    CallRange range_("shampoo4_refresh_root");
    if (!c) return SHAMPOO4_EINVAL;
    hipStream_t s = as_stream(stream);
    hipError_t e = c->debug_fill(s);
    if (e == hipSuccess) e = c->run(c->root_d, s);
    if (e == hipSuccess) e = c->run(c->root_copy, s);
    if (e == hipSuccess && (c->cfg.flags & SHAMPOO4_FLAG_ROOT_CACHE)) {
        e = c->root_eigenvectors(s);
        c->root_v_valid = (e == hipSuccess);
        c->root_v_is_stats = (e == hipSuccess);
    } else {
        c->root_v_valid = false;
    }
    return e == hipSuccess ? SHAMPOO4_OK : SHAMPOO4_EHIP;
}

shampoo4_status shampoo4_precondition(shampoo4_ctx c, const shampoo4_io* io, void* stream) {
    CallRange range_("shampoo4_precondition");
    if (!c) return SHAMPOO4_EINVAL;
    shampoo4_status st = validate_io(c, io, true);
    if (st != SHAMPOO4_OK) return st;
    hipStream_t s = as_stream(stream);
    if (c->debug_fill(s) != hipSuccess) return SHAMPOO4_EHIP;
    if (c->upload_io(io, s) != hipSuccess) return SHAMPOO4_EHIP;
    hipError_t e = hipSuccess;
    if (!((c->cfg.flags & SHAMPOO4_FLAG_ROOT_CACHE) && c->root_v_valid)) {
        e = c->root_eigenvectors(s);
        c->root_v_is_stats = false;
    }
    if (c->cfg.flags & SHAMPOO4_FLAG_ROOT_CACHE) {
        for (int i = 0; i < 2 && e == hipSuccess; ++i) e = c->run(c->pre_cached[i], s);
    } else {
        for (int i = 0; i < 4 && e == hipSuccess; ++i) e = c->run(c->pre[i], s);
    }
    if (e == hipSuccess) e = c->run(c->diag_pre, s);
    return e == hipSuccess ? SHAMPOO4_OK : SHAMPOO4_EHIP;
}

shampoo4_status shampoo4_step(shampoo4_ctx c, const shampoo4_io* io, int32_t refresh, void* stream) {
    CallRange range_("shampoo4_step");
    if (!c) return SHAMPOO4_EINVAL;
    shampoo4_status st = validate_io(c, io, true);
    if (st != SHAMPOO4_OK) return st;
    // (batches large enough for the blocked QR keep the GPU busy by themselves: there
    // the three parts run in order)
    const bool overlap = !refresh && (c->cfg.flags & SHAMPOO4_FLAG_ROOT_CACHE) && c->root_v_valid &&
                         c->outer == kPanel;
    if (!overlap) {
        st = shampoo4_update_stats(c, io, stream);
        if (st == SHAMPOO4_OK && refresh) st = shampoo4_refresh_root(c, stream);
        if (st == SHAMPOO4_OK) st = shampoo4_precondition(c, io, stream);
        return st;
    }
    // P = Rt_L G Rt_R reads only the cached root matrices, G and its own temporaries,
    // none of which the statistics update touches: it runs on a second stream (default
    // priority) beside the statistics chain, from where that chain's QR begins (its
    // panels leave most CUs idle).
    hipStream_t s = as_stream(stream);
    if (c->ensure_pre_stream() != hipSuccess) return SHAMPOO4_EHIP;
    if (c->debug_fill(s) != hipSuccess) return SHAMPOO4_EHIP;
    if (c->upload_io(io, s) != hipSuccess) return SHAMPOO4_EHIP;
    // the precondition is enqueued at the fork point itself (host order), so its launches
    // reach the GPU as the QR starts rather than after the host has queued the whole chain
    const std::function<hipError_t()> fork = [c, s]() {
        hipError_t e = hipEventRecord(c->pre_fork, s);
        if (e == hipSuccess) e = hipStreamWaitEvent(c->pre_strm, c->pre_fork, 0);
        for (int i = 0; i < 2 && e == hipSuccess; ++i) e = c->run(c->pre_side[i], c->pre_strm);
        if (e == hipSuccess) e = c->run(c->diag_pre, c->pre_strm);
        if (e == hipSuccess) e = hipEventRecord(c->pre_join, c->pre_strm);
        return e;
    };
    hipError_t e = c->submit_stats(s, &fork);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, c->pre_join, 0);
    return e == hipSuccess ? SHAMPOO4_OK : SHAMPOO4_EHIP;
}

shampoo4_status shampoo4_graft(shampoo4_ctx c, const shampoo4_io* io, const shampoo4_graft_io* gio,
                               const shampoo4_graft_config* cfg, void* stream) {
    CallRange range_("shampoo4_graft");
    if (!c || !gio || !cfg) return SHAMPOO4_EINVAL;
    shampoo4_status st = validate_io(c, io, true);
    if (st != SHAMPOO4_OK) return st;
    if (cfg->mode != SHAMPOO4_GRAFT_SGD && cfg->mode != SHAMPOO4_GRAFT_ADAM) return SHAMPOO4_EINVAL;
    if (!std::isfinite(cfg->lr) || !(cfg->eps_graft >= 0.f) || !std::isfinite(cfg->eps_graft))
        return SHAMPOO4_EINVAL;
    const bool adam = cfg->mode == SHAMPOO4_GRAFT_ADAM;
    if (adam && (cfg->step < 1 || !(cfg->beta1 >= 0.f && cfg->beta1 < 1.f) ||
                 !(cfg->beta2 >= 0.f && cfg->beta2 < 1.f) || !(cfg->eps_adam >= 0.f) ||
                 !std::isfinite(cfg->eps_adam)))
        return SHAMPOO4_EINVAL;
    for (int b = 0; b < c->nb; ++b) {
        if (!gio[b].W || (adam && (!gio[b].M || !gio[b].V))) return SHAMPOO4_EINVAL;
        if (gio[b].ldw < c->shapes[b].n) return SHAMPOO4_ESHAPE;
    }
    GraftParams prm{};
    prm.mode = adam ? 1 : 0;
    prm.lr = cfg->lr;
    prm.eps_graft = cfg->eps_graft;
    prm.beta1 = cfg->beta1;
    prm.beta2 = cfg->beta2;
    prm.eps_adam = cfg->eps_adam;
    prm.c1 = adam ? (float)(1.0 - std::pow((double)cfg->beta1, (double)cfg->step)) : 1.f;
    prm.c2 = adam ? (float)(1.0 - std::pow((double)cfg->beta2, (double)cfg->step)) : 1.f;
    if (adam && !(prm.c1 > 0.f && prm.c2 > 0.f)) return SHAMPOO4_EINVAL;
    c->graft_prm = prm;
    hipStream_t s = as_stream(stream);
    if (c->debug_fill(s) != hipSuccess) return SHAMPOO4_EHIP;
    if (c->upload_io(io, s) != hipSuccess) return SHAMPOO4_EHIP;
    if (c->upload_table(gio, c->gio_off, s) != hipSuccess) return SHAMPOO4_EHIP;
    const hipError_t e = c->run(c->graft_seq[prm.mode], s);
    return e == hipSuccess ? SHAMPOO4_OK : SHAMPOO4_EHIP;
}

shampoo4_status shampoo4_check(shampoo4_ctx c, void* stream, uint32_t* device_flags) {
    CallRange range_("shampoo4_check");
    if (!c) return SHAMPOO4_EINVAL;
    hipStream_t s = as_stream(stream);
    uint32_t f = 0;
    if (hipStreamSynchronize(s) != hipSuccess) return SHAMPOO4_EHIP;
    if (hipMemcpy(&f, c->ws + c->flag_off, sizeof(f), hipMemcpyDeviceToHost) != hipSuccess)
        return SHAMPOO4_EHIP;
    if (device_flags) *device_flags = f;
    if (f) {
        const uint32_t zero = 0;
        if (hipMemcpy(c->ws + c->flag_off, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
            return SHAMPOO4_EHIP;
        return SHAMPOO4_ENONFINITE;
    }
    return SHAMPOO4_OK;
}

shampoo4_status shampoo4_destroy(shampoo4_ctx c) {
    if (!c) return SHAMPOO4_EINVAL;
    for (int i = 0; i < kRing; ++i)
        if (c->ring_used[i]) (void)hipEventSynchronize(c->ring_ev[i]);
    delete c;
    return SHAMPOO4_OK;
}

shampoo4_status shampoo4_layout(shampoo4_ctx c, int32_t block, int32_t side, shampoo4_buffer which,
                                size_t* offset, size_t* bytes) {
    if (!c || !offset || !bytes) return SHAMPOO4_EINVAL;
    if (block < 0 || block >= c->nb || side < 0 || side > 1) return SHAMPOO4_EINVAL;
    const Side& S = c->sides[2 * block + side];
    const size_t p = S.p;
    const size_t mat = p * p * 4;
    if (S.diag && which >= SHAMPOO4_BUF_V) return SHAMPOO4_EINVAL;   // a diagonal side has no matrices
    // the float64 update keeps its statistic and eigenvectors in float64 (and no float32 V)
    if (c->fp64 && (which == SHAMPOO4_BUF_V || which == SHAMPOO4_BUF_STAT)) return SHAMPOO4_EINVAL;
    if (!c->fp64 && (which == SHAMPOO4_BUF_STAT64 || which == SHAMPOO4_BUF_Q64)) return SHAMPOO4_EINVAL;
    switch (which) {
        case SHAMPOO4_BUF_CODES: *offset = S.codes; *bytes = c->fp32_state ? (size_t)p * p * 4 : S.nqb * 32; break;
        case SHAMPOO4_BUF_SCALES: *offset = S.scales; *bytes = c->fp32_state ? 0 : S.nqb * 4; break;
        case SHAMPOO4_BUF_EIG: *offset = S.lam; *bytes = p * 4; break;
        case SHAMPOO4_BUF_ROOT_CODES: *offset = S.rcodes; *bytes = c->fp32_state ? (size_t)p * p * 4 : S.nqb * 32; break;
        case SHAMPOO4_BUF_ROOT_SCALES: *offset = S.rscales; *bytes = c->fp32_state ? 0 : S.nqb * 4; break;
        case SHAMPOO4_BUF_ROOT_D: *offset = S.d; *bytes = p * 4; break;
        case SHAMPOO4_BUF_V: *offset = S.Vs; *bytes = mat; break;
        case SHAMPOO4_BUF_STAT: *offset = S.Lt; *bytes = mat; break;
        case SHAMPOO4_BUF_Q: *offset = S.Qm; *bytes = mat; break;
        case SHAMPOO4_BUF_ROOT_V: *offset = S.Vr; *bytes = mat; break;
        case SHAMPOO4_BUF_ROOT_MAT: *offset = S.Rt; *bytes = mat; break;
        case SHAMPOO4_BUF_STAT64: *offset = S.Lt64; *bytes = 2 * mat; break;
        case SHAMPOO4_BUF_Q64: *offset = S.Q64; *bytes = 2 * mat; break;
        default: return SHAMPOO4_EINVAL;
    }
    return SHAMPOO4_OK;
}

shampoo4_status shampoo4_codebook_ex(int32_t codebook, float levels[16], float midpoints[15]) {
    if (!levels || !midpoints) return SHAMPOO4_EINVAL;
    return host_codebook(codebook, levels, midpoints) ? SHAMPOO4_OK : SHAMPOO4_EINVAL;
}

shampoo4_status shampoo4_codebook(float levels[16], float midpoints[15]) {
    return shampoo4_codebook_ex(SHAMPOO4_CODEBOOK_LINEAR_SQUARE, levels, midpoints);
}

static bool valid_codebook(int32_t codebook) {
    return codebook == SHAMPOO4_CODEBOOK_LINEAR_SQUARE || codebook == SHAMPOO4_CODEBOOK_DYNAMIC_TREE;
}

shampoo4_status shampoo4_quantize(const float* x, int64_t n, int32_t qblock, uint8_t* codes, float* scales,
                                  void* stream) {
    return shampoo4_quantize_ex(x, n, qblock, SHAMPOO4_CODEBOOK_LINEAR_SQUARE, codes, scales, stream);
}

shampoo4_status shampoo4_dequantize(const uint8_t* codes, const float* scales, int64_t n, int32_t qblock,
                                    float* x, void* stream) {
    return shampoo4_dequantize_ex(codes, scales, n, qblock, SHAMPOO4_CODEBOOK_LINEAR_SQUARE, x, stream);
}

shampoo4_status shampoo4_quantize_ex(const float* x, int64_t n, int32_t qblock, int32_t codebook, uint8_t* codes,
                                     float* scales, void* stream) {
    CallRange range_("shampoo4_quantize_ex");
    if (qblock != 64 || n < 0 || !valid_codebook(codebook)) return SHAMPOO4_EINVAL;
    if (n == 0) return SHAMPOO4_OK;
    if (!x || !codes || !scales) return SHAMPOO4_EINVAL;
    if ((reinterpret_cast<uintptr_t>(codes) & 1) || (reinterpret_cast<uintptr_t>(scales) & 3) ||
        (reinterpret_cast<uintptr_t>(x) & 3))
        return SHAMPOO4_EALIGN;
    CodecDesc d;
    std::memset(&d, 0, sizeof(d));
    d.x_in = x; d.codes_out = codes; d.scales_out = scales; d.n = n;
    return launch_quant_single(codebook, d, as_stream(stream)) == hipSuccess ? SHAMPOO4_OK : SHAMPOO4_EHIP;
}

shampoo4_status shampoo4_dequantize_ex(const uint8_t* codes, const float* scales, int64_t n, int32_t qblock,
                                       int32_t codebook, float* x, void* stream) {
    CallRange range_("shampoo4_dequantize_ex");
    if (qblock != 64 || n < 0 || !valid_codebook(codebook)) return SHAMPOO4_EINVAL;
    if (n == 0) return SHAMPOO4_OK;
    if (!x || !codes || !scales) return SHAMPOO4_EINVAL;
    if ((reinterpret_cast<uintptr_t>(codes) & 3) || (reinterpret_cast<uintptr_t>(scales) & 3) ||
        (reinterpret_cast<uintptr_t>(x) & 3))
        return SHAMPOO4_EALIGN;
    CodecDesc d;
    std::memset(&d, 0, sizeof(d));
    d.codes_in = codes; d.scales_in = scales; d.x_out = x; d.n = n;
    return launch_dequant_single(codebook, d, as_stream(stream)) == hipSuccess ? SHAMPOO4_OK : SHAMPOO4_EHIP;
}

size_t shampoo4_gemm_workspace_bytes(int32_t count) {
    return align_up((size_t)std::max(count, 0) * sizeof(GemmDesc)) + align_up(((size_t)std::max(count, 0) + 1) * 4);
}

}  // extern "C"

namespace {

// Validates a batched product and plans its single launch: `tmp.blob` then holds the
// descriptor table and tile prefix (offsets in `L` relative to the blob's start); `L.ntiles`
// is 0 when there is nothing to compute.
shampoo4_status plan_gemm_batched(int32_t kernel, int32_t count, int32_t transA, int32_t transB, const int32_t* M,
                                  const int32_t* N, const int32_t* K, float alpha, const float* const* A,
                                  const int64_t* lda, const float* const* B, const int64_t* ldb, float beta,
                                  const float* const* C, const int64_t* ldc, float* const* D, const int64_t* ldd,
                                  shampoo4_ctx_s& tmp, Launch& L) {
    L = Launch{};
    if (kernel != SHAMPOO4_GEMM_AUTO && kernel != SHAMPOO4_GEMM_FP32 && kernel != SHAMPOO4_GEMM_X3)
        return SHAMPOO4_EINVAL;
    tmp.x3 = kernel != SHAMPOO4_GEMM_FP32;
    if (count < 0) return SHAMPOO4_EINVAL;
    if (count == 0) return SHAMPOO4_OK;
    if (!M || !N || !K || !A || !lda || !B || !ldb || !D || !ldd) return SHAMPOO4_EINVAL;
    if (beta != 0.f && (!C || !ldc)) return SHAMPOO4_EINVAL;
    std::vector<shampoo4_ctx_s::GemmItem> items;
    for (int i = 0; i < count; ++i) {
        if (M[i] < 0 || N[i] < 0 || K[i] < 0) return SHAMPOO4_ESHAPE;
        const int64_t acols = transA ? M[i] : K[i];
        const int64_t bcols = transB ? K[i] : N[i];
        const bool empty_out = M[i] == 0 || N[i] == 0;
        if ((!empty_out && !D[i]) || (!empty_out && K[i] > 0 && (!A[i] || !B[i]))) return SHAMPOO4_EINVAL;
        if (lda[i] < std::max<int64_t>(acols, 1) || ldb[i] < std::max<int64_t>(bcols, 1) ||
            ldd[i] < std::max<int32_t>(N[i], 1))
            return SHAMPOO4_ESHAPE;
        if (beta != 0.f && (!C[i] || ldc[i] < std::max<int32_t>(N[i], 1))) return SHAMPOO4_ESHAPE;
        GemmDesc d = tmp.gd(A[i], lda[i], B[i], ldb[i], D[i], ldd[i], M[i], N[i], K[i], alpha, beta,
                            beta != 0.f ? C[i] : nullptr, beta != 0.f ? ldc[i] : 0);
        items.push_back({d, transA != 0, transB != 0});
    }
    // one launch: one descriptor table and one tile prefix (the tile shape follows the
    // products' class when they all share one)
    Seq seq = kernel == SHAMPOO4_GEMM_X3 ? tmp.gemm_launch(items, FAM_GEMM_PRECOND, GEMM_128x128)
                                         : tmp.make_gemm(items, FAM_GEMM_PRECOND);
    if (seq.size() > 1) {
        tmp.blob.clear();
        seq = tmp.make_gemm(items, FAM_GEMM_PRECOND, false, false);
    }
    if (!seq.empty()) L = seq[0];
    return SHAMPOO4_OK;
}

// Copies the planned table to `dev` (device memory) and launches the product on it.
shampoo4_status run_gemm_batched(const shampoo4_ctx_s& tmp, const Launch& L, uint8_t* dev, hipStream_t s) {
    if (hipMemcpyAsync(dev, tmp.blob.data(), tmp.blob.size(), hipMemcpyHostToDevice, s) != hipSuccess)
        return SHAMPOO4_EHIP;
    hipError_t e = launch_gemm(L.cfg, L.mode, L.vec, L.slab, L.kscale, reinterpret_cast<const GemmDesc*>(dev + L.desc_off),
                               reinterpret_cast<const int*>(dev + L.prefix_off), L.ndesc, L.ntiles, nullptr, s);
    return e == hipSuccess ? SHAMPOO4_OK : SHAMPOO4_EHIP;
}

}  // namespace

extern "C" {

shampoo4_status shampoo4_gemm_batched(int32_t count, int32_t transA, int32_t transB, const int32_t* M,
                                      const int32_t* N, const int32_t* K, float alpha, const float* const* A,
                                      const int64_t* lda, const float* const* B, const int64_t* ldb, float beta,
                                      const float* const* C, const int64_t* ldc, float* const* D,
                                      const int64_t* ldd, void* workspace, size_t workspace_bytes,
                                      void* stream) {
    return shampoo4_gemm_batched_ex(SHAMPOO4_GEMM_AUTO, count, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta,
                                    C, ldc, D, ldd, workspace, workspace_bytes, stream);
}

shampoo4_status shampoo4_gemm_batched_ex(int32_t kernel, int32_t count, int32_t transA, int32_t transB,
                                         const int32_t* M, const int32_t* N, const int32_t* K, float alpha,
                                         const float* const* A, const int64_t* lda, const float* const* B,
                                         const int64_t* ldb, float beta, const float* const* C, const int64_t* ldc,
                                         float* const* D, const int64_t* ldd, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    CallRange range_("shampoo4_gemm_batched_ex");
    if (count > 0) {
        if (!workspace) return SHAMPOO4_EINVAL;
        if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return SHAMPOO4_EALIGN;
        if (workspace_bytes < shampoo4_gemm_workspace_bytes(count)) return SHAMPOO4_ESMALLBUF;
    }
    shampoo4_ctx_s tmp;
    Launch L;
    shampoo4_status st = plan_gemm_batched(kernel, count, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                           ldc, D, ldd, tmp, L);
    if (st != SHAMPOO4_OK || L.ntiles <= 0) return st;
    // the descriptors and their tile prefix sit at the start of the caller's workspace
    if (tmp.blob.size() > workspace_bytes) return SHAMPOO4_ESMALLBUF;
    return run_gemm_batched(tmp, L, static_cast<uint8_t*>(workspace), as_stream(stream));
}

shampoo4_status shampoo4_gemm_batched_static(int32_t count, int32_t transA, int32_t transB, const int32_t* M,
                                             const int32_t* N, const int32_t* K, float alpha,
                                             const float* const* A, const int64_t* lda, const float* const* B,
                                             const int64_t* ldb, float beta, const float* const* C,
                                             const int64_t* ldc, float* const* D, const int64_t* ldd,
                                             void* stream) {
    CallRange range_("shampoo4_gemm_batched_static");
    if (count > SHAMPOO4_GEMM_STATIC_MAX) return SHAMPOO4_ESMALLBUF;
    shampoo4_ctx_s tmp;
    Launch L;
    shampoo4_status st = plan_gemm_batched(SHAMPOO4_GEMM_AUTO, count, transA, transB, M, N, K, alpha, A, lda, B, ldb,
                                           beta, C, ldc, D, ldd, tmp, L);
    if (st != SHAMPOO4_OK || L.ntiles <= 0) return st;
    if (tmp.blob.size() > GEMM_STATIC_SCRATCH_BYTES) return SHAMPOO4_ESMALLBUF;
    void* scr = nullptr;   // this device's array (its address looked up at the first call)
    if (gemm_static_scratch(&scr) != hipSuccess) return SHAMPOO4_EHIP;
    return run_gemm_batched(tmp, L, static_cast<uint8_t*>(scr), as_stream(stream));
}

namespace {

// Plan of one coupled Newton call over caller-given matrices: work buffers first, then
// the descriptor tables; `ctx.ws` must already point at the workspace (or null for sizing).
struct NewtonPlan {
    shampoo4_ctx_s ctx;
    size_t buffers = 0;
    Seq seq;
};

void plan_newton(NewtonPlan& np, int32_t count, const int32_t* p, const float* const* A, const int64_t* lda,
                 int32_t iters, float* const* X, const int64_t* ldx) {
    shampoo4_ctx_s& c = np.ctx;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes ? bytes : 1); return o; };
    struct Bufs { size_t M[2], X[2], F, F2, F4, parts, scale; };
    std::vector<Bufs> bufs(count);
    for (int i = 0; i < count; ++i) {
        const size_t mat = (size_t)p[i] * p[i] * 4;
        Bufs& b = bufs[i];
        b.M[0] = take(mat); b.M[1] = take(mat); b.X[0] = take(mat); b.X[1] = take(mat);
        b.F = take(mat); b.F2 = take(mat); b.F4 = take(mat);
        b.parts = take((size_t)fill_tiles(p[i]) * 4);
        b.scale = take(4);
    }
    np.buffers = off;
    c.desc_base = off;
    c.blob.clear();
    auto wf = [&](size_t o) { return c.wsf(o); };
    std::vector<NewtonDesc> base(count);
    std::vector<int> tiles(count);
    for (int i = 0; i < count; ++i) {
        NewtonDesc d;
        std::memset(&d, 0, sizeof(d));
        d.A = A ? A[i] : nullptr; d.lda = lda ? lda[i] : 0;
        d.out = X ? X[i] : nullptr; d.ldo = ldx ? ldx[i] : 0;
        d.parts = wf(bufs[i].parts); d.scale = wf(bufs[i].scale);
        d.p = p[i];
        base[i] = d;
        tiles[i] = fill_tiles(p[i]);
    }
    auto elem = [&](int mode, auto fill) {
        std::vector<NewtonDesc> ds = base;
        for (int i = 0; i < count; ++i) fill(ds[i], bufs[i]);
        Launch L = c.make_items(K_NEWTON_ELEM, ds, tiles);
        L.mode = mode;
        return L;
    };
    np.seq.clear();
    np.seq.push_back(c.make_items(K_NEWTON_NORM, base, tiles));
    {
        std::vector<int> ones(count, 1);
        np.seq.push_back(c.make_items(K_NEWTON_SCALE, base, ones));
    }
    np.seq.push_back(elem(0, [&](NewtonDesc& d, const Bufs& b) { d.dst = wf(b.M[0]); d.ident = wf(b.X[0]); }));
    Seq per[2];
    for (int q = 0; q < 2; ++q) {
        per[q].push_back(elem(1, [&](NewtonDesc& d, const Bufs& b) { d.src = wf(b.M[q]); d.dst = wf(b.F); }));
        std::vector<shampoo4_ctx_s::GemmItem> g1, g2, g3;
        for (int i = 0; i < count; ++i) {
            const int n = p[i];
            const Bufs& b = bufs[i];
            g1.push_back({c.gd(wf(b.X[q]), n, wf(b.F), n, wf(b.X[1 - q]), n, n, n, n), false, false});
            g1.push_back({c.gd(wf(b.F), n, wf(b.F), n, wf(b.F2), n, n, n, n), false, false});
            g2.push_back({c.gd(wf(b.F2), n, wf(b.F2), n, wf(b.F4), n, n, n, n), false, false});
            g3.push_back({c.gd(wf(b.F4), n, wf(b.M[q]), n, wf(b.M[1 - q]), n, n, n, n), false, false});
        }
        for (auto* items : {&g1, &g2, &g3}) {
            Seq g = c.make_gemm(*items, FAM_GEMM_PRECOND);
            per[q].insert(per[q].end(), g.begin(), g.end());
        }
    }
    for (int it = 0; it < iters; ++it) np.seq.insert(np.seq.end(), per[it & 1].begin(), per[it & 1].end());
    np.seq.push_back(elem(2, [&](NewtonDesc& d, const Bufs& b) { d.src = wf(b.X[iters & 1]); }));
}

}  // namespace

size_t shampoo4_inverse_root_workspace_bytes(int32_t count, const int32_t* p) {
    if (count <= 0 || !p) return 0;
    for (int i = 0; i < count; ++i)
        if (p[i] < 1 || p[i] > kMaxDim) return 0;
    NewtonPlan np;
    plan_newton(np, count, p, nullptr, nullptr, 2, nullptr, nullptr);
    return np.buffers + align_up(np.ctx.blob.size());
}

shampoo4_status shampoo4_inverse_root(int32_t count, const int32_t* p, const float* const* A, const int64_t* lda,
                                      float eps, int32_t iters, float* const* X, const int64_t* ldx,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    CallRange range_("shampoo4_inverse_root");
    if (count < 0) return SHAMPOO4_EINVAL;
    if (count == 0) return SHAMPOO4_OK;
    if (!p || !A || !lda || !X || !ldx || !workspace) return SHAMPOO4_EINVAL;
    if (!(eps >= 0.f) || !std::isfinite(eps) || iters < 0 || iters > 100) return SHAMPOO4_EINVAL;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return SHAMPOO4_EALIGN;
    for (int i = 0; i < count; ++i) {
        if (p[i] < 1 || p[i] > kMaxDim) return SHAMPOO4_ESHAPE;
        if (!A[i] || !X[i]) return SHAMPOO4_EINVAL;
        if (lda[i] < p[i] || ldx[i] < p[i]) return SHAMPOO4_ESHAPE;
    }
    if (workspace_bytes < shampoo4_inverse_root_workspace_bytes(count, p)) return SHAMPOO4_ESMALLBUF;
    NewtonPlan np;
    np.ctx.ws = static_cast<uint8_t*>(workspace);
    np.ctx.newton_eps = eps;
    plan_newton(np, count, p, A, lda, iters, X, ldx);
    hipStream_t s = as_stream(stream);
    if (hipMemcpyAsync(np.ctx.ws + np.ctx.desc_base, np.ctx.blob.data(), np.ctx.blob.size(),
                       hipMemcpyHostToDevice, s) != hipSuccess)
        return SHAMPOO4_EHIP;
    return np.ctx.run(np.seq, s) == hipSuccess ? SHAMPOO4_OK : SHAMPOO4_EHIP;
}

shampoo4_status shampoo4_timing(shampoo4_ctx c, int32_t enable) {
    if (!c) return SHAMPOO4_EINVAL;
    c->timing = enable != 0;
    c->recs.clear();
    c->ev_used = 0;
    return SHAMPOO4_OK;
}

shampoo4_status shampoo4_timing_report(shampoo4_ctx c, int32_t* count, const char** names, int64_t* launches,
                                       double* total_ms, double* flops, double* bytes) {
    if (!c || !count) return SHAMPOO4_EINVAL;
    if (*count < FAM_N || !names || !launches || !total_ms || !flops || !bytes) {
        *count = FAM_N;
        return SHAMPOO4_EINVAL;
    }
    for (int f = 0; f < FAM_N; ++f) {
        names[f] = kFamilyNames[f];
        launches[f] = 0;
        total_ms[f] = flops[f] = bytes[f] = 0;
    }
    for (auto& r : c->recs) {
        if (hipEventSynchronize(r.e1) != hipSuccess) return SHAMPOO4_EHIP;
        float ms = 0;
        if (hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess) return SHAMPOO4_EHIP;
        launches[r.family] += 1;
        total_ms[r.family] += ms;
        flops[r.family] += r.flops;
        bytes[r.family] += r.bytes;
        if (r.x3) {
            launches[FAM_GEMM_X3] += 1;
            total_ms[FAM_GEMM_X3] += ms;
            flops[FAM_GEMM_X3] += r.flops;
            bytes[FAM_GEMM_X3] += r.bytes;
        }
    }
    *count = FAM_N;
    return SHAMPOO4_OK;
}

}  // extern "C"
