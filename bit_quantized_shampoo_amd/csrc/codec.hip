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
//    the group writes the scale.
//  * dequant: one lane per 8 elements (one 32-bit code word, two 16-byte
//    stores), levels looked up in a 16-entry LDS table (conflict-free).
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

__device__ __forceinline__ uint32_t code_of(float xh) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 15; ++j) c += (xh > kMid[j]) ? 1u : 0u;
    return c;
}

__device__ __forceinline__ void dequant_item(const CodecDesc& d, int tile) {
    __shared__ float lv[16];
    if (threadIdx.x < 16) lv[threadIdx.x] = c_levels[threadIdx.x];
    __syncthreads();
    const int64_t w = (int64_t)tile * 256 + threadIdx.x;
    const int64_t n = d.n;
    const int64_t nwords = ((n + 63) / 64) * 8;
    if (w >= nwords) return;
    const uint32_t cw = reinterpret_cast<const uint32_t*>(d.codes_in)[w];
    const float s = d.scales_in[w >> 3];
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = lv[(cw >> (4 * e)) & 15u] * s;
    const int64_t e0 = w * 8;
    float* __restrict__ x = d.x_out;
    if (e0 + 8 <= n && ((reinterpret_cast<uintptr_t>(x) & 15) == 0)) {
        floatx4 a = {v[0], v[1], v[2], v[3]};
        floatx4 b = {v[4], v[5], v[6], v[7]};
        *reinterpret_cast<floatx4*>(x + e0) = a;
        *reinterpret_cast<floatx4*>(x + e0 + 4) = b;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e0 + e < n) x[e0 + e] = v[e];
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

__device__ __forceinline__ void quant_item(const CodecDesc& d, int tile, uint32_t* __restrict__ flag) {
    const int64_t qd = (int64_t)tile * 256 + threadIdx.x;
    const int64_t n = d.n;
    const int64_t nquads = ((n + 63) / 64) * 16;
    const bool active = qd < nquads;
    const float* __restrict__ x = d.x_in;
    const int64_t e0 = qd * 4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (active) {
        if (e0 + 4 <= n && ((reinterpret_cast<uintptr_t>(x) & 15) == 0)) {
            const floatx4 q = *reinterpret_cast<const floatx4*>(x + e0);
            v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e0 + e < n) v[e] = x[e0 + e];
        }
    }
    bool finite = true;
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        finite = finite && __builtin_isfinite(v[e]);
        amax = fmaxf(amax, fabsf(v[e]));
    }
    // absmax over the 16 lanes of this quantization block (lane groups are aligned)
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    if (!active) return;
    if (!finite && flag) flag[0] = 1u;
    uint32_t packed;
    if (amax == 0.f) {
        packed = 0x7777u;
    } else {
        packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) packed |= code_of(__fdiv_rn(v[e], amax)) << (4 * e);
    }
    reinterpret_cast<uint16_t*>(d.codes_out)[qd] = (uint16_t)packed;
    if ((qd & 15) == 0) d.scales_out[qd >> 4] = amax;
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
    hipLaunchKernelGGL(dequant_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc);
    return hipGetLastError();
}

hipError_t launch_quant(const CodecDesc* descs, const int* prefix, int ndesc, int ntiles,
                        uint32_t* flag, hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(quant_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc, flag);
    return hipGetLastError();
}

hipError_t launch_dequant_single(const CodecDesc& d, hipStream_t stream) {
    const int64_t tiles = ((d.n + 63) / 64 * 8 + 255) / 256;
    if (tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_single_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, d);
    return hipGetLastError();
}

hipError_t launch_quant_single(const CodecDesc& d, hipStream_t stream) {
    const int64_t tiles = ((d.n + 63) / 64 * 16 + 255) / 256;
    if (tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(quant_single_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, d);
    return hipGetLastError();
}

hipError_t launch_codec_copy(const CodecDesc* descs, const int* prefix, int ndesc, int ntiles,
                             hipStream_t stream) {
    if (ntiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(codec_copy_kernel, dim3(ntiles), dim3(256), 0, stream, descs, prefix, ndesc);
    return hipGetLastError();
}

}  // namespace s4
