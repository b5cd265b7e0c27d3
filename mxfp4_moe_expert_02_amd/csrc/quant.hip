// quant.hip -- MXFP4 and MXFP8 weight encoders, gfx950.
//
// MXFP4 encoding of float32 weights along the rows, one thread per
// block of 32 (OCP MX block: 32 E2M1 elements + one E8M0 scale), the format
// the pages give the expert weights (bjdmk.com.cn page, 4 bits per
// parameter).  The element rounding is written as a count of crossed
// midpoints, each compare choosing the side that keeps ties on the even code.
// The MXFP8 encoder (E4M3 elements) is for the weights that stay at 8 bits
// beside the 4-bit experts (the optional shared expert).
#include "mx_encode.h"

namespace moe {
namespace {

// floor(log2(a)) of a finite a > 0 given as float bits
__device__ inline int floor_log2_f32(uint32_t bits) {
    int ef = (int)(bits >> 23) & 0xff;
    if (ef) return ef - 127;
    uint32_t m = bits & 0x7fffffu;  // subnormal: value m * 2^-149
    return (31 - __clz((int)m)) - 149;
}

// nearest E2M1 magnitude code of a >= 0, ties to even code, saturating at 6
__device__ inline uint32_t e2m1_code(float a) {
    return (uint32_t)(a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
           (a >= 3.5f) + (a > 5.0f);
}

constexpr int kQuantThreads = 256;

__global__ void __launch_bounds__(kQuantThreads)
quantize_mxfp4_kernel(const float* __restrict__ w, int64_t nblocks, int64_t blocks_per_row,
                      int64_t cols, uint8_t* __restrict__ packed, uint8_t* __restrict__ scales) {
    const int64_t b = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    if (b >= nblocks) return;
    const int64_t r = b / blocks_per_row, c = b % blocks_per_row;
    const float4* src = reinterpret_cast<const float4*>(w + r * cols + c * 32);
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        float4 q = src[i];
        v[4 * i] = q.x;
        v[4 * i + 1] = q.y;
        v[4 * i + 2] = q.z;
        v[4 * i + 3] = q.w;
    }
    uint32_t amax_bits = 0;
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 32; i++) {
        uint32_t a = __float_as_uint(v[i]) & 0x7fffffffu;
        finite = finite && (a < 0x7f800000u);
        amax_bits = a > amax_bits ? a : amax_bits;  // |x| order == bit order for finite x
    }
    uint4 out = make_uint4(0, 0, 0, 0);
    uint8_t sc;
    if (!finite) {
        sc = 255;
    } else {
        int se = (amax_bits == 0) ? -127 : floor_log2_f32(amax_bits) - 2;
        se = se < -127 ? -127 : (se > 127 ? 127 : se);
        sc = (uint8_t)(se + 127);
        uint32_t words[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 32; i++) {
            float q = ldexpf(v[i], -se);  // exact scaling by a power of two
            uint32_t code = e2m1_code(fabsf(q)) | ((__float_as_uint(q) >> 28) & 8u);
            words[i / 8] |= code << (4 * (i % 8));
        }
        out = make_uint4(words[0], words[1], words[2], words[3]);
    }
    *reinterpret_cast<uint4*>(packed + r * (cols / 2) + c * 16) = out;
    scales[r * blocks_per_row + c] = sc;
}

// MXFP8 encoding of float32 weights: one thread per block of 32
__global__ void __launch_bounds__(kQuantThreads)
quantize_mxfp8_kernel(const float* __restrict__ w, int64_t nblocks, uint8_t* __restrict__ codes,
                      uint8_t* __restrict__ scales) {
    const int64_t b = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    if (b >= nblocks) return;
    const float4* src = reinterpret_cast<const float4*>(w + b * 32);
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float4 q = src[i];
        v[4 * i] = q.x;
        v[4 * i + 1] = q.y;
        v[4 * i + 2] = q.z;
        v[4 * i + 3] = q.w;
    }
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 32; i++) {
        const uint32_t m = __float_as_uint(v[i]) & 0x7fffffffu;
        amax = m > amax ? m : amax;  // NaN and infinity bits order above every finite value
    }
    uint32_t c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint8_t s = 255;
    if (amax < 0x7f800000u) {
        const int se = mxfp8_scale_exp(amax);
        s = (uint8_t)(se + 127);
#pragma unroll
        for (int i = 0; i < 32; i++) c[i / 4] |= e4m3_code(v[i], se) << (8 * (i % 4));
    }
    uint4* dst = reinterpret_cast<uint4*>(codes + b * 32);
    dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
    dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
    scales[b] = s;
}

}  // namespace

hipError_t launch_quantize_mxfp8(const float* w, int64_t rows, int64_t cols, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream) {
    const int64_t nblocks = rows * (cols / 32);
    if (nblocks == 0) return hipSuccess;
    quantize_mxfp8_kernel<<<(unsigned)((nblocks + kQuantThreads - 1) / kQuantThreads), kQuantThreads,
                            0, stream>>>(w, nblocks, codes, scales);
    return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(const float* w, int64_t rows, int64_t cols, uint8_t* packed,
                                 uint8_t* scales, hipStream_t stream) {
    int64_t bpr = cols / 32;
    int64_t nblocks = rows * bpr;
    if (nblocks == 0) return hipSuccess;
    int64_t grid = (nblocks + kQuantThreads - 1) / kQuantThreads;
    quantize_mxfp4_kernel<<<(unsigned)grid, kQuantThreads, 0, stream>>>(w, nblocks, bpr, cols,
                                                                         packed, scales);
    return hipGetLastError();
}

}  // namespace moe
