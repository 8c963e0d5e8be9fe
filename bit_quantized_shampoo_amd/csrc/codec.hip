// Block-wise 4-bit codecs ("4-bit Shampoo for Memory-Efficient Network Training",
// abstract: the eigenvector matrix is stored in 4 bits, block-wise, with linear-square
// quantization, which the abstract compares with dynamic tree quantization).
//
// Linear-square codebook: 16 levels sign(t) t^2 on the grid t = -1 + 2j/15 (j = 0..15)
// with the j = 7 level set to an exact zero; times 225 the levels are
//   -225 -169 -121 -81 -49 -25 -9 0 1 9 25 49 81 121 169 225.
// Dynamic tree codebook (defined in the 8-bit optimizers paper the pages cite): a sign
// bit and three magnitude bits whose leading zeros E are a base-10 exponent, then an
// indicator bit and 2 - E linear fraction bits (midpoints of equal bins of [0.1, 1],
// times 10^-E); zero, and +1 in place of the negative zero so that a block's maximum is
// exact.  Ascending, times 2000:
//   -1775 -1325 -875 -425 -155 -65 -11 0 11 65 155 425 875 1325 1775 2000.
// Codes index the ascending levels (the zero level is code 7 in both).  A value x of a
// 64-element block with absmax s > 0 is normalized as x_hat = x / s (IEEE correctly
// rounded) and coded as the number of float32 decision midpoints strictly below x_hat
// (a value equal to a midpoint takes the lower code); s = 0 codes the whole block as
// the zero level.  Two codes per byte, even element in the low nibble.
// Dequantization is one fp32 multiply q[code] * s.
//
// Both kernels are HBM-bound streams: the quantizer reads 4 B and writes
// 0.5 B + 4/64 B per element, the dequantizer the reverse.
//  * quant: one lane per 4 consecutive elements (a 16-byte load), 16 lanes per
//    block; the block absmax is a 4-step DPP reduction inside the 16-lane row;
//    x_hat comes from one correctly rounded reciprocal per block and two fused
//    multiply-add corrections per element (bit-identical to the IEEE division);
//    each lane writes its 4 codes as one 16-bit store, lane 0 of the group
//    writes the scale.  The code comes from one LDS table lookup keyed by the
//    bits of x_hat instead of a scan over the 15 midpoints.
//  * dequant: a lane expands 4 elements at a time (one 16-bit code word, one
//    16-byte store), several quads per lane in flight, spaced so that every store
//    instruction of a wave writes 1 KB contiguous; levels from a 16-entry LDS table.
#include "kernels.hpp"

namespace s4 {

namespace {

// Level numerators over DEN, ascending.  Levels and midpoints are rounded once to
// fp32 from double (a host test checks them bit-for-bit against exactly rounded
// values).  MB: mantissa bits of the quantizer's bucket key (below).
struct LinearSquare {
    static constexpr int ID = SHAMPOO4_CODEBOOK_LINEAR_SQUARE;
    static constexpr double DEN = 225.0;
    static constexpr int NUM[16] = {-225, -169, -121, -81, -49, -25, -9, 0, 1, 9, 25, 49, 81, 121, 169, 225};
    static constexpr int MB = 2;
};
struct DynamicTree {
    static constexpr int ID = SHAMPOO4_CODEBOOK_DYNAMIC_TREE;
    static constexpr double DEN = 2000.0;
    static constexpr int NUM[16] = {-1775, -1325, -875, -425, -155, -65, -11, 0,
                                    11,    65,    155,  425,  875,  1325, 1775, 2000};
    static constexpr int MB = 3;
};

template <class CB> constexpr float level_of(int j) { return (float)((double)CB::NUM[j] / CB::DEN); }
template <class CB> constexpr float mid_of(int j) {
    return (float)((double)(CB::NUM[j] + CB::NUM[j + 1]) / (2.0 * CB::DEN));
}

__constant__ float c_levels[2][16] = {
    {level_of<LinearSquare>(0), level_of<LinearSquare>(1), level_of<LinearSquare>(2), level_of<LinearSquare>(3),
     level_of<LinearSquare>(4), level_of<LinearSquare>(5), level_of<LinearSquare>(6), level_of<LinearSquare>(7),
     level_of<LinearSquare>(8), level_of<LinearSquare>(9), level_of<LinearSquare>(10), level_of<LinearSquare>(11),
     level_of<LinearSquare>(12), level_of<LinearSquare>(13), level_of<LinearSquare>(14), level_of<LinearSquare>(15)},
    {level_of<DynamicTree>(0), level_of<DynamicTree>(1), level_of<DynamicTree>(2), level_of<DynamicTree>(3),
     level_of<DynamicTree>(4), level_of<DynamicTree>(5), level_of<DynamicTree>(6), level_of<DynamicTree>(7),
     level_of<DynamicTree>(8), level_of<DynamicTree>(9), level_of<DynamicTree>(10), level_of<DynamicTree>(11),
     level_of<DynamicTree>(12), level_of<DynamicTree>(13), level_of<DynamicTree>(14), level_of<DynamicTree>(15)}};

// Code lookup without a midpoint scan.  The magnitude's float32 bit pattern, shifted
// right by 23 - MB, is the exponent with the top MB mantissa bits: a bucket of width at
// most (1 + 2^-MB)x.  Adjacent midpoints of one sign differ by at least 1.36x
// (linear-square, MB = 2: buckets of 1.25x) or 1.21x (dynamic tree, MB = 3: 1.125x), so
// every bucket over [2^-9, 2) holds at most one midpoint (checked at compile time
// below) and magnitudes under 2^-9 lie below every midpoint.  Each (sign, bucket) entry
// stores the code of a magnitude at or below the bucket's midpoint, the code above it,
// and the midpoint's bit pattern as an unsigned threshold; the result equals the count
// of midpoints strictly below x_hat for every float32 x_hat, signed zeros and
// subnormals included.
constexpr uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

template <class CB>
struct Buckets {
    static constexpr int SHIFT = 23 - CB::MB;
    static constexpr int E0 = 118 << CB::MB;   // bucket 0 starts at 2^-9 (biased exponent 118)
    static constexpr int N = 10 << CB::MB;     // buckets per sign, [2^-9, 2)
    static constexpr int bucket_of(uint32_t mag) {
        const int b = (int)(mag >> SHIFT) - E0;
        return b < 0 ? 0 : (b >= N ? N - 1 : b);
    }
};

template <class CB>
struct QTab {
    uint32_t thr[2 * Buckets<CB>::N];    // the in-bucket midpoint (as x_hat bits), or all ones
    uint32_t code[2 * Buckets<CB>::N];   // low nibble: code at or below thr; next nibble: code above
    int max_per_bucket;
    bool mids_in_range;                  // every midpoint magnitude lies in [2^-9, 2)
};

template <class CB>
constexpr QTab<CB> make_qtab() {
    using B = Buckets<CB>;
    QTab<CB> t{};
    t.max_per_bucket = 0;
    t.mids_in_range = true;
    int negatives = 0;
    for (int j = 0; j < 15; ++j) {
        const uint32_t mag = f32_bits(mid_of<CB>(j)) & 0x7fffffffu;
        const int raw = (int)(mag >> B::SHIFT) - B::E0;
        if (raw < 0 || raw >= B::N) t.mids_in_range = false;
        if (mid_of<CB>(j) < 0.0f) ++negatives;
    }
    if (negatives != 7) t.mids_in_range = false;   // the zero level must be code 7
    for (int s = 0; s < 2; ++s) {
        for (int b = 0; b < B::N; ++b) {
            const uint32_t lo_u = b > 0 ? (uint32_t)(b + B::E0) << B::SHIFT : 0u;
            int below = 0, inb = 0;
            uint32_t thr = 0xffffffffu;
            for (int j = 0; j < 15; ++j) {
                const bool neg = mid_of<CB>(j) < 0.0f;
                if (neg != (s == 1)) continue;
                const uint32_t mag = f32_bits(mid_of<CB>(j)) & 0x7fffffffu;
                if (mag < lo_u) ++below;
                if (B::bucket_of(mag) == b) {
                    ++inb;
                    // positive: code rises once x_hat > m; negative: the count of
                    // midpoints below x_hat drops once |x_hat| >= |m|.  The threshold is
                    // compared with x_hat's whole bit pattern, so a negative entry
                    // carries the sign bit.
                    thr = s == 0 ? mag : ((mag - 1u) | 0x80000000u);
                }
            }
            const int lo = s == 0 ? 7 + below : 7 - below;
            const int hi = inb ? (s == 0 ? lo + 1 : lo - 1) : lo;
            t.thr[s * B::N + b] = thr;
            t.code[s * B::N + b] = (uint32_t)lo | ((uint32_t)hi << 4);
            if (inb > t.max_per_bucket) t.max_per_bucket = inb;
        }
    }
    return t;
}

constexpr QTab<LinearSquare> kQTabLS = make_qtab<LinearSquare>();
constexpr QTab<DynamicTree> kQTabDT = make_qtab<DynamicTree>();
static_assert(kQTabLS.max_per_bucket == 1 && kQTabDT.max_per_bucket == 1,
              "a code bucket holds more than one midpoint");
static_assert(kQTabLS.mids_in_range && kQTabDT.mids_in_range,
              "a midpoint lies outside the buckets (or the zero level is not code 7)");

__constant__ QTab<LinearSquare> c_qtab_ls = kQTabLS;
__constant__ QTab<DynamicTree> c_qtab_dt = kQTabDT;

template <class CB> __device__ __forceinline__ const QTab<CB>& qtab();
template <> __device__ __forceinline__ const QTab<LinearSquare>& qtab<LinearSquare>() { return c_qtab_ls; }
template <> __device__ __forceinline__ const QTab<DynamicTree>& qtab<DynamicTree>() { return c_qtab_dt; }

template <class CB>
__device__ __forceinline__ uint32_t code_of(float xh, const uint2* __restrict__ tab) {
    using B = Buckets<CB>;
    const uint32_t u = __float_as_uint(xh);
    // exponent and top MB mantissa bits of |x_hat| (one bit-field extract), clamped to
    // the bucket range (one med3)
    const uint32_t key = min(max(__builtin_amdgcn_ubfe(u, B::SHIFT, 31 - B::SHIFT), (uint32_t)B::E0),
                             (uint32_t)(B::E0 + B::N - 1));
    const uint2 e = tab[(int)key - B::E0 + (int)(u >> 31) * B::N];
    return __builtin_amdgcn_ubfe(e.y, u > e.x ? 4u : 0u, 4u);
}

// Dequantization: each lane expands DEQ_QUADS groups of 4 elements (one 16-bit code
// word, one 16-byte store) spaced 256 quads apart, so every store instruction of a wave
// writes 1 KB contiguous.
constexpr int DEQ_QUADS = DEQ_TILE / (256 * 4);

template <class CB>
__device__ __forceinline__ void dequant_item(const CodecDesc& d, int tile) {
    __shared__ float lv[16];
    if (threadIdx.x < 16) lv[threadIdx.x] = c_levels[CB::ID][threadIdx.x];
    __syncthreads();
    const int64_t n = d.n;
    const int64_t nquads = ((n + 63) / 64) * 16;
    const int64_t q0 = (int64_t)tile * (DEQ_TILE / 4) + threadIdx.x;
    const uint16_t* __restrict__ cq = reinterpret_cast<const uint16_t*>(d.codes_in);
    uint32_t cw[DEQ_QUADS];
    float sc[DEQ_QUADS];
#pragma unroll
    for (int k = 0; k < DEQ_QUADS; ++k) {
        const int64_t q = min(q0 + k * 256, nquads - 1);
        cw[k] = ldg(cq + q);
        sc[k] = ldg(d.scales_in + (q >> 4));
    }
    float* __restrict__ x = d.x_out;
    const bool aligned = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
#pragma unroll
    for (int k = 0; k < DEQ_QUADS; ++k) {
        const int64_t q = q0 + k * 256;
        if (q >= nquads) break;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = lv[(cw[k] >> (4 * e)) & 15u] * sc[k];
        const int64_t e0 = q * 4;
        if (e0 + 4 <= n && aligned) {
            const floatx4 a = {v[0], v[1], v[2], v[3]};
            stg_nt(reinterpret_cast<floatx4*>(x + e0), a);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e0 + e < n) x[e0 + e] = v[e];
        }
    }
}

template <class CB>
__global__ __launch_bounds__(256) void dequant_kernel(const CodecDesc* __restrict__ descs,
                                                      const int* __restrict__ prefix, int ndesc) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    dequant_item<CB>(descs[item], blockIdx.x - prefix[item]);
}

template <class CB>
__global__ __launch_bounds__(256) void dequant_single_kernel(CodecDesc d) {
    dequant_item<CB>(d, blockIdx.x);
}

// Quantization: a lane codes 4 consecutive elements (one 16-byte load), 16 lanes (one
// DPP row) cover a quantization block; each lane handles QUANT_QUADS such quads spaced
// 256 quads apart.  The block absmax is taken on the magnitudes' bit patterns (as
// unsigned integers they order like the floats, and NaN / Inf sort above every finite
// value, so the same maximum flags non-finite input) and reduced over the row with
// four DPP rotations.
constexpr int QUANT_QUADS = QUANT_TILE / (256 * 4);

// Largest value over the 16 lanes of a DPP row: rotations by 8, 4, 2, 1 reach every lane.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t m) {
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x128, 0xf, 0xf, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x124, 0xf, 0xf, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x122, 0xf, 0xf, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x121, 0xf, 0xf, false));
    return m;
}

// x / s rounded to nearest from y = RN(1/s), without a division per element.  The first
// correction q1 = q0 + (x - q0 s) y leaves q1 within one ulp of x / s; the second is
// Markstein's correction step: when y = RN(1/s) and q is within one ulp of x / s, the
// remainder x - q s is exact in one fused multiply-add and RN(q + (x - q s) y) = RN(x / s).
// Its conditions (no underflow of the remainders where the quotient can reach a decision
// midpoint, |x/s| >= 2^-9) hold for 2^-60 <= s <= 2^60; a quotient below 2^-12 lies below
// every midpoint however it is rounded.  Other scales take the IEEE division.
constexpr uint32_t kRecipLo = 0x21800000u;   // 2^-60
constexpr uint32_t kRecipHi = 0x5d800000u;   // 2^60
__device__ __forceinline__ float quotient_rn(float x, float s, float y) {
    const float q0 = x * y;
    const float q1 = fmaf(fmaf(-q0, s, x), y, q0);
    return fmaf(fmaf(-q1, s, x), y, q1);
}

template <class CB>
__device__ __forceinline__ void quant_item(const CodecDesc& d, int tile, uint32_t* __restrict__ flag) {
    constexpr int NT = 2 * Buckets<CB>::N;
    static_assert(NT <= 256, "one table entry per thread");
    __shared__ uint2 tab[NT];
    if (threadIdx.x < NT) tab[threadIdx.x] = make_uint2(qtab<CB>().thr[threadIdx.x], qtab<CB>().code[threadIdx.x]);
    const int64_t n = d.n;
    const int64_t nquads = ((n + 63) / 64) * 16;
    const int64_t q0 = (int64_t)tile * (QUANT_TILE / 4) + threadIdx.x;
    const float* __restrict__ x = d.x_in;
    const bool aligned = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
    // every element of the tile exists: straight-line streaming loads
    const bool full = aligned && (int64_t)(tile + 1) * QUANT_TILE <= n;
    float v[QUANT_QUADS][4];
    if (full) {
#pragma unroll
        for (int k = 0; k < QUANT_QUADS; ++k) {
            const floatx4 q = ldg_nt(reinterpret_cast<const floatx4*>(x + (q0 + k * 256) * 4));
            v[k][0] = q[0]; v[k][1] = q[1]; v[k][2] = q[2]; v[k][3] = q[3];
        }
    } else {
#pragma unroll
        for (int k = 0; k < QUANT_QUADS; ++k) {
            const int64_t e0 = (q0 + k * 256) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[k][e] = 0.f;
            if (e0 + 4 <= n && aligned) {
                const floatx4 q = ldg_nt(reinterpret_cast<const floatx4*>(x + e0));
                v[k][0] = q[0]; v[k][1] = q[1]; v[k][2] = q[2]; v[k][3] = q[3];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (e0 + e < n) v[k][e] = ldg(x + e0 + e);
            }
        }
    }
    __syncthreads();
    uint32_t bad = 0;
#pragma unroll
    for (int k = 0; k < QUANT_QUADS; ++k) {
        const int64_t qd = q0 + k * 256;
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) m = max(m, __float_as_uint(v[k][e]) & 0x7fffffffu);
        m = row_max_u32(m);
        bad |= m >= 0x7f800000u ? 1u : 0u;
        const float amax = __uint_as_float(m);
        if (qd < nquads) {
            uint32_t packed = 0;
            if (m >= kRecipLo && m <= kRecipHi) {
                const float y = __fdiv_rn(1.0f, amax);
#pragma unroll
                for (int e = 0; e < 4; ++e) packed |= code_of<CB>(quotient_rn(v[k][e], amax, y), tab) << (4 * e);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) packed |= code_of<CB>(__fdiv_rn(v[k][e], amax), tab) << (4 * e);
                if (m == 0u) packed = 0x7777u;
            }
            reinterpret_cast<uint16_t*>(d.codes_out)[qd] = (uint16_t)packed;
            if ((qd & 15) == 0) d.scales_out[qd >> 4] = amax;
        }
    }
    if (bad && flag) flag[0] = 1u;
}

template <class CB>
__global__ __launch_bounds__(256) void quant_kernel(const CodecDesc* __restrict__ descs,
                                                    const int* __restrict__ prefix, int ndesc,
                                                    uint32_t* __restrict__ flag) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    quant_item<CB>(descs[item], blockIdx.x - prefix[item], flag);
}

template <class CB>
__global__ __launch_bounds__(256) void quant_single_kernel(CodecDesc d) {
    quant_item<CB>(d, blockIdx.x, nullptr);
}

// Copy of codes and scales (root snapshot).
__global__ __launch_bounds__(256) void codec_copy_kernel(const CodecDesc* __restrict__ descs,
                                                         const int* __restrict__ prefix, int ndesc) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    const CodecDesc& d = descs[item];
    const int64_t nqb = (d.n + 63) / 64;
    const int64_t nvec = nqb * 2;      // 16-byte chunks of codes (32 bytes per block)
    const int64_t base = (int64_t)(blockIdx.x - prefix[item]) * (COPY_TILE / 16);
    for (int64_t i = base + threadIdx.x; i < base + COPY_TILE / 16 && i < nvec; i += 256) {
        reinterpret_cast<uint4*>(d.codes_out)[i] = reinterpret_cast<const uint4*>(d.codes_in)[i];
    }
    const int64_t sbase = (int64_t)(blockIdx.x - prefix[item]) * (COPY_TILE / 32);
    for (int64_t i = sbase + threadIdx.x; i < sbase + COPY_TILE / 32 && i < nqb; i += 256)
        d.scales_out[i] = d.scales_in[i];
}

}  // namespace

template <class CB>
void fill_codebook(float levels[16], float midpoints[15]) {
    for (int i = 0; i < 16; ++i) levels[i] = level_of<CB>(i);
    for (int i = 0; i < 15; ++i) midpoints[i] = mid_of<CB>(i);
}

bool host_codebook(int codebook, float levels[16], float midpoints[15]) {
    if (codebook == LinearSquare::ID) fill_codebook<LinearSquare>(levels, midpoints);
    else if (codebook == DynamicTree::ID) fill_codebook<DynamicTree>(levels, midpoints);
    else return false;
    return true;
}

hipError_t launch_dequant(int codebook, const CodecDesc* descs, const int* prefix, int ndesc, int ntiles,
                          hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    if (codebook == DynamicTree::ID)
        S4_LAUNCH(dequant_kernel<DynamicTree>, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc);
    else
        S4_LAUNCH(dequant_kernel<LinearSquare>, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc);
    return hipGetLastError();
}

hipError_t launch_quant(int codebook, const CodecDesc* descs, const int* prefix, int ndesc, int ntiles,
                        uint32_t* flag, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    if (codebook == DynamicTree::ID)
        S4_LAUNCH(quant_kernel<DynamicTree>, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, flag);
    else
        S4_LAUNCH(quant_kernel<LinearSquare>, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, flag);
    return hipGetLastError();
}

hipError_t launch_dequant_single(int codebook, const CodecDesc& d, hipStream_t stream) {
    const int64_t tiles = dequant_tiles(d.n);
    if (tiles <= 0) return hipSuccess;
    if (codebook == DynamicTree::ID)
        S4_LAUNCH(dequant_single_kernel<DynamicTree>, dim3((unsigned)tiles), dim3(256), 0, stream, d);
    else
        S4_LAUNCH(dequant_single_kernel<LinearSquare>, dim3((unsigned)tiles), dim3(256), 0, stream, d);
    return hipGetLastError();
}

hipError_t launch_quant_single(int codebook, const CodecDesc& d, hipStream_t stream) {
    const int64_t tiles = quant_tiles(d.n);
    if (tiles <= 0) return hipSuccess;
    if (codebook == DynamicTree::ID)
        S4_LAUNCH(quant_single_kernel<DynamicTree>, dim3((unsigned)tiles), dim3(256), 0, stream, d);
    else
        S4_LAUNCH(quant_single_kernel<LinearSquare>, dim3((unsigned)tiles), dim3(256), 0, stream, d);
    return hipGetLastError();
}

hipError_t launch_codec_copy(const CodecDesc* descs, const int* prefix, int ndesc, int ntiles,
                             hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(codec_copy_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc);
    return hipGetLastError();
}

}  // namespace s4
