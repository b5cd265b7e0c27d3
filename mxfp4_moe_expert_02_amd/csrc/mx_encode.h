// mx_encode.h -- MXFP8 (E4M3 elements, one E8M0 scale per block of 32)
// encoding helpers shared by the activation and weight encoders: the OCP
// MX block rule, scale 2^(floor(log2 amax) - 8) (8 = the exponent of the
// largest E4M3 value, 448), elements rounded to the nearest E4M3 value with
// ties to the even code, saturating at 448.
#pragma once

#include "moe_internal.h"

namespace moe {

// nearest E4M3 (OCP FN) magnitude code of a >= 0: ties to the even code,
// saturating at 448 (code 126); subnormals below 2^-6 in steps of 2^-9
__device__ inline uint32_t e4m3_mag_code(float a) {
    if (!(a < 448.f)) return 126u;
    if (a < 0.015625f) return (uint32_t)rintf(a * 512.f);
    const int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;  // floor(log2 a)
    const uint32_t t = (uint32_t)rintf(ldexpf(a, 3 - e));             // 8..16
    const uint32_t code = (uint32_t)((e + 7) << 3) + t - 8u;          // t = 16 carries into e+1
    return code > 126u ? 126u : code;
}

// floor(log2(a)) of a finite a > 0 given as float bits
__device__ inline int floor_log2_bits(uint32_t bits) {
    const int ef = (int)(bits >> 23) & 0xff;
    if (ef) return ef - 127;
    return (31 - __clz((int)(bits & 0x7fffffu))) - 149;
}

// Block scale exponent of the MXFP8 rule from the block's largest |v| as
// float bits: floor(log2 amax) - 8, clamped to [-127, 127]; amax == 0 gives
// -127.  amax_bits >= 0x7f800000 (a NaN or an infinity in the block) is the
// caller's case: scale 0xFF, codes 0.
__device__ inline int mxfp8_scale_exp(uint32_t amax_bits) {
    const int se = amax_bits == 0 ? -127 : floor_log2_bits(amax_bits) - 8;
    return se < -127 ? -127 : (se > 127 ? 127 : se);
}

// E4M3 code (sign included) of v / 2^se
__device__ inline uint32_t e4m3_code(float v, int se) {
    const float q = ldexpf(v, -se);  // exact: a power-of-two scaling
    return e4m3_mag_code(fabsf(q)) | ((__float_as_uint(q) >> 24) & 0x80u);
}

}  // namespace moe
