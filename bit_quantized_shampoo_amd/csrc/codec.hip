// Block-wise 4-bit linear-square codec ("4-bit Shampoo for Memory-Efficient Network
// Training", abstract: the eigenvector matrix is stored in 4 bits with linear-square
// quantization, block-wise).
//
// Codebook: 16 levels sign(t) t^2 on the grid t = -1 + 2j/15 (j = 0..15) with the
// j = 7 level set to an exact zero; times 225 the levels are
//   -225 -169 -121 -81 -49 -25 -9 0 1 9 25 49 81 121 169 225.
// A value x of a 64-element block with absmax s > 0 is normalized as
// x_hat = x / s (IEEE correctly rounded) and coded as the number of float32
// decision midpoints strictly below x_hat (a value equal to a midpoint takes the
// lower code); s = 0 codes the whole block as the zero level.  Two codes per byte,
// even element in the low nibble.  Dequantization is one fp32 multiply q[code] * s.
//
// Both kernels are HBM-bound streams: the quantizer reads 4 B and writes
// 0.5 B + 4/64 B per element, the dequantizer the reverse.
//  * quant: one lane per 4 consecutive elements (a 16-byte load), 16 lanes per
//    block; the block absmax is a 4-step xor-shuffle reduction inside the
//    16-lane group; each lane writes its 4 codes as one 16-bit store, lane 0 of
//    the group writes the scale.  The code comes from one LDS table lookup keyed
//    by the bits of x_hat instead of a scan over the 15 midpoints.
//  * dequant: a lane expands 4 elements at a time (one 16-bit code word, one
//    16-byte store), several quads per lane in flight, spaced so that every store
//    instruction of a wave writes 1 KB contiguous; levels from a 16-entry LDS table.
#include "kernels.hpp"

namespace s4 {

namespace {

// Level numerators over 225 and midpoint numerators over 450, rounded once to fp32
// from double (a host test checks them bit-for-bit against exactly rounded values).
#define S4_LV(a) ((float)((double)(a) / 225.0))
#define S4_MP(a, b) ((float)((double)((a) + (b)) / 450.0))

__constant__ float c_levels[16] = {
    S4_LV(-225), S4_LV(-169), S4_LV(-121), S4_LV(-81), S4_LV(-49), S4_LV(-25), S4_LV(-9), 0.0f,
    S4_LV(1),    S4_LV(9),    S4_LV(25),   S4_LV(49),  S4_LV(81),  S4_LV(121), S4_LV(169), S4_LV(225)};

constexpr float kMid[15] = {
    S4_MP(-225, -169), S4_MP(-169, -121), S4_MP(-121, -81), S4_MP(-81, -49), S4_MP(-49, -25),
    S4_MP(-25, -9),    S4_MP(-9, 0),      S4_MP(0, 1),      S4_MP(1, 9),     S4_MP(9, 25),
    S4_MP(25, 49),     S4_MP(49, 81),     S4_MP(81, 121),   S4_MP(121, 169), S4_MP(169, 225)};

constexpr float kLevelsHost[16] = {
    S4_LV(-225), S4_LV(-169), S4_LV(-121), S4_LV(-81), S4_LV(-49), S4_LV(-25), S4_LV(-9), 0.0f,
    S4_LV(1),    S4_LV(9),    S4_LV(25),   S4_LV(49),  S4_LV(81),  S4_LV(121), S4_LV(169), S4_LV(225)};

// Code lookup without a midpoint scan.  The magnitude's float32 bit pattern, shifted
// right by 21, is the exponent with the top two mantissa bits: a bucket of width at
// most 1.25x.  Adjacent midpoints of one sign differ by at least 1.36x, so every
// bucket over [2^-9, 2) holds at most one midpoint (checked at compile time below)
// and magnitudes under 2^-9 lie below every midpoint.  Each (sign, bucket) entry
// stores the code of a magnitude at or below the bucket's midpoint, the code above
// it, and the midpoint's bit pattern as an unsigned threshold; the result equals the
// count of midpoints strictly below x_hat for every float32 x_hat, signed zeros and
// subnormals included.
constexpr uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }
constexpr int QB_E0 = 118 * 4;   // bucket 0 starts at 2^-9 (biased exponent 118)
constexpr int QB_N = 40;         // buckets per sign, [2^-9, 2)

constexpr int bucket_of(uint32_t mag) {
    const int b = (int)(mag >> 21) - QB_E0;
    return b < 0 ? 0 : (b >= QB_N ? QB_N - 1 : b);
}

struct QTab {
    uint32_t thr[2 * QB_N];    // the in-bucket midpoint (as magnitude bits), or all ones
    uint32_t code[2 * QB_N];   // low nibble: code at or below thr; next nibble: code above
    int max_per_bucket;
};

constexpr QTab make_qtab() {
    QTab t{};
    t.max_per_bucket = 0;
    for (int s = 0; s < 2; ++s) {
        for (int b = 0; b < QB_N; ++b) {
            const uint32_t lo_u = b > 0 ? (uint32_t)(b + QB_E0) << 21 : 0u;
            int below = 0, inb = 0;
            uint32_t thr = 0xffffffffu;
            for (int j = 0; j < 15; ++j) {
                const bool neg = kMid[j] < 0.0f;
                if (neg != (s == 1)) continue;
                const uint32_t mag = f32_bits(kMid[j]) & 0x7fffffffu;
                if (mag < lo_u) ++below;
                if (bucket_of(mag) == b) {
                    ++inb;
                    // positive: code rises once x_hat > m; negative: the count of
                    // midpoints below x_hat drops once |x_hat| >= |m|
                    thr = s == 0 ? mag : mag - 1u;
                }
            }
            const int lo = s == 0 ? 7 + below : 7 - below;
            const int hi = inb ? (s == 0 ? lo + 1 : lo - 1) : lo;
            t.thr[s * QB_N + b] = thr;
            t.code[s * QB_N + b] = (uint32_t)lo | ((uint32_t)hi << 4);
            if (inb > t.max_per_bucket) t.max_per_bucket = inb;
        }
    }
    return t;
}

constexpr QTab kQTab = make_qtab();
static_assert(kQTab.max_per_bucket == 1, "a code bucket holds more than one midpoint");
static_assert(f32_bits(kMid[7]) >> 21 >= QB_E0 && (f32_bits(-kMid[6]) >> 21) >= QB_E0,
              "a midpoint lies below the first bucket");

__constant__ QTab c_qtab = kQTab;

__device__ __forceinline__ uint32_t code_of(float xh, const uint2* __restrict__ tab) {
    const uint32_t u = __float_as_uint(xh);
    const uint32_t mag = u & 0x7fffffffu;
    const int b = min(max((int)(mag >> 21) - QB_E0, 0), QB_N - 1) + (int)(u >> 31) * QB_N;
    const uint2 e = tab[b];
    return mag > e.x ? (e.y >> 4) : (e.y & 15u);
}

// Dequantization: each lane expands DEQ_QUADS groups of 4 elements (one 16-bit code
// word, one 16-byte store) spaced 256 quads apart, so every store instruction of a wave
// writes 1 KB contiguous.
constexpr int DEQ_QUADS = DEQ_TILE / (256 * 4);

__device__ __forceinline__ void dequant_item(const CodecDesc& d, int tile) {
    __shared__ float lv[16];
    if (threadIdx.x < 16) lv[threadIdx.x] = c_levels[threadIdx.x];
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
            stg(reinterpret_cast<floatx4*>(x + e0), a);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e0 + e < n) x[e0 + e] = v[e];
        }
    }
}

__global__ __launch_bounds__(256) void dequant_kernel(const CodecDesc* __restrict__ descs,
                                                      const int* __restrict__ prefix, int ndesc) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    dequant_item(descs[item], blockIdx.x - prefix[item]);
}

__global__ __launch_bounds__(256) void dequant_single_kernel(CodecDesc d) {
    dequant_item(d, blockIdx.x);
}

// Quantization: a lane codes 4 consecutive elements (one 16-byte load), 16 lanes
// cover a quantization block and reduce its absmax with xor shuffles; each lane
// handles QUANT_QUADS such quads spaced 256 quads apart.
constexpr int QUANT_QUADS = QUANT_TILE / (256 * 4);

__device__ __forceinline__ void quant_item(const CodecDesc& d, int tile, uint32_t* __restrict__ flag) {
    __shared__ uint2 tab[2 * QB_N];
    if (threadIdx.x < 2 * QB_N) tab[threadIdx.x] = make_uint2(c_qtab.thr[threadIdx.x], c_qtab.code[threadIdx.x]);
    const int64_t n = d.n;
    const int64_t nquads = ((n + 63) / 64) * 16;
    const int64_t q0 = (int64_t)tile * (QUANT_TILE / 4) + threadIdx.x;
    const float* __restrict__ x = d.x_in;
    const bool aligned = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
    float v[QUANT_QUADS][4];
#pragma unroll
    for (int k = 0; k < QUANT_QUADS; ++k) {
        const int64_t e0 = (q0 + k * 256) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[k][e] = 0.f;
        if (e0 + 4 <= n && aligned) {
            const floatx4 q = *reinterpret_cast<const floatx4*>(x + e0);
            v[k][0] = q[0]; v[k][1] = q[1]; v[k][2] = q[2]; v[k][3] = q[3];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e0 + e < n) v[k][e] = x[e0 + e];
        }
    }
    __syncthreads();
    bool finite = true;
#pragma unroll
    for (int k = 0; k < QUANT_QUADS; ++k) {
        const int64_t qd = q0 + k * 256;
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            finite = finite && __builtin_isfinite(v[k][e]);
            amax = fmaxf(amax, fabsf(v[k][e]));
        }
        // absmax over the 16 lanes of this quantization block (lane groups are aligned)
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
        if (qd < nquads) {
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) packed |= code_of(__fdiv_rn(v[k][e], amax), tab) << (4 * e);
            if (amax == 0.f) packed = 0x7777u;
            reinterpret_cast<uint16_t*>(d.codes_out)[qd] = (uint16_t)packed;
            if ((qd & 15) == 0) d.scales_out[qd >> 4] = amax;
        }
    }
    if (!finite && flag) flag[0] = 1u;
}

__global__ __launch_bounds__(256) void quant_kernel(const CodecDesc* __restrict__ descs,
                                                    const int* __restrict__ prefix, int ndesc,
                                                    uint32_t* __restrict__ flag) {
    const int item = find_item(prefix, ndesc, blockIdx.x);
    quant_item(descs[item], blockIdx.x - prefix[item], flag);
}

__global__ __launch_bounds__(256) void quant_single_kernel(CodecDesc d) {
    quant_item(d, blockIdx.x, nullptr);
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

void host_codebook(float levels[16], float midpoints[15]) {
    for (int i = 0; i < 16; ++i) levels[i] = kLevelsHost[i];
    for (int i = 0; i < 15; ++i) midpoints[i] = kMid[i];
}

hipError_t launch_dequant(const CodecDesc* descs, const int* prefix, int ndesc, int ntiles,
                          hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(dequant_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc);
    return hipGetLastError();
}

hipError_t launch_quant(const CodecDesc* descs, const int* prefix, int ndesc, int ntiles,
                        uint32_t* flag, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(quant_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, flag);
    return hipGetLastError();
}

hipError_t launch_dequant_single(const CodecDesc& d, hipStream_t stream) {
    const int64_t tiles = dequant_tiles(d.n);
    if (tiles <= 0) return hipSuccess;
    S4_LAUNCH(dequant_single_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, d);
    return hipGetLastError();
}

hipError_t launch_quant_single(const CodecDesc& d, hipStream_t stream) {
    const int64_t tiles = quant_tiles(d.n);
    if (tiles <= 0) return hipSuccess;
    S4_LAUNCH(quant_single_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, d);
    return hipGetLastError();
}

hipError_t launch_codec_copy(const CodecDesc* descs, const int* prefix, int ndesc, int ntiles,
                             hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    S4_LAUNCH(codec_copy_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc);
    return hipGetLastError();
}

}  // namespace s4
