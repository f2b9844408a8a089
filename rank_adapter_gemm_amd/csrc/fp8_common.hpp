// E4M3 quantization helpers shared by the FP8 quantizers and the fused
// quantize-and-shrink of decode rows: power-of-two scales and the codes.
#pragma once

#include "common.hpp"

namespace lora {

constexpr float kE4M3Max = 448.0f;

// Exponent of the power-of-two scale of a row or column whose largest
// magnitude is amax (>= 0, finite): the smallest e with amax <= 448 * 2^e,
// clamped to [-127, 127].  With amax = m 2^E (1 <= m < 2) and 448 = 1.75 2^8:
// e = E - 8 if m <= 1.75, else E - 7; zero and subnormal amax give -127.
__device__ __forceinline__ int scale_exp(float amax) {
    const uint32_t u = __float_as_uint(amax);
    const int field = (int)(u >> 23);
    if (field == 0) return -127;
    const int e = field - 135 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
    return e < -127 ? -127 : e;
}

// 2^e as an fp32 value, exactly, for e in [-127, 127] (2^-127 is subnormal).
__device__ __forceinline__ float exp2i(int e) {
    return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// E8M0 code (biased exponent) of a power-of-two scale 2^e, e in [-127, 127].
__device__ __forceinline__ int e8m0_of(float s) { return (int)((__float_as_uint(s) >> 23) & 0xffu); }

// Four fp32 values (already scaled) to four E4M3 codes, byte i = value i.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
    b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
    c = fminf(fmaxf(c, -kE4M3Max), kE4M3Max);
    d = fminf(fmaxf(d, -kE4M3Max), kE4M3Max);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

}  // namespace lora
