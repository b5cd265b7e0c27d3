// combine_quant.hip -- the weighted combine of expert outputs and the MXFP4
// weight encoder, gfx950.
//
// combine: out[t] = sum_j w[t,j] * y[pos[t,j]], summed in slot order j =
// 0..k-1 in fp32 and rounded to bf16 (nearest even).  A gather, not a
// scatter: no atomics, so the result is bit-reproducible.  This realises the
// weighted sum of the k experts' outputs that top-k MoE routing implies
// (bjdmk.com.cn news page, co-design section: each expert sees only part of
// the tokens).
//
// quantize: MXFP4 encoding of float32 weights along the rows, one thread per
// block of 32 (OCP MX block: 32 E2M1 elements + one E8M0 scale), the format
// the pages give the expert weights (bjdmk.com.cn page, 4 bits per
// parameter).  The element rounding is written as a count of crossed
// midpoints, each compare choosing the side that keeps ties on the even code.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

constexpr int kCombineThreads = 256;

// grid (ceil(H / (4*256)), T); each thread owns 4 consecutive columns
__global__ void __launch_bounds__(kCombineThreads)
combine_kernel(const float* __restrict__ y, const float* __restrict__ wts,
               const int32_t* __restrict__ pos, int H, int k, uint16_t* __restrict__ out) {
    const int t = blockIdx.y;
    const int n = (blockIdx.x * kCombineThreads + threadIdx.x) * 4;
    if (n >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; j++) {
        float w = wts[(int64_t)t * k + j];
        int p = pos[(int64_t)t * k + j];
        float4 v = *reinterpret_cast<const float4*>(y + (int64_t)p * H + n);
        acc.x = fmaf(w, v.x, acc.x);
        acc.y = fmaf(w, v.y, acc.y);
        acc.z = fmaf(w, v.z, acc.z);
        acc.w = fmaf(w, v.w, acc.w);
    }
    ushort4 o;
    o.x = f32_to_bf16_rne(acc.x);
    o.y = f32_to_bf16_rne(acc.y);
    o.z = f32_to_bf16_rne(acc.z);
    o.w = f32_to_bf16_rne(acc.w);
    *reinterpret_cast<ushort4*>(out + (int64_t)t * H + n) = o;
}

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

}  // namespace

hipError_t launch_combine(const float* y, const float* wts, const int32_t* pos, int T, int H,
                          int k, uint16_t* out, hipStream_t stream) {
    dim3 grid((H / 4 + kCombineThreads - 1) / kCombineThreads, T);
    combine_kernel<<<grid, kCombineThreads, 0, stream>>>(y, wts, pos, H, k, out);
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
