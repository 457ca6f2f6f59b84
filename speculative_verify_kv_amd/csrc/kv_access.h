// Device helpers: element conversions and paged-cache addressing (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swattn {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// float -> bfloat16 bits, round to nearest even, NaN kept NaN (hardware cvt on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    __bf16 h = (__bf16)x;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// OCP E4M3 code -> its value times 2^-8, exactly.
//
// The 7 magnitude bits of an E4M3 code, shifted left by 7, form an IEEE half
// whose exponent field is the E4M3 exponent field and whose top 3 mantissa bits
// are the E4M3 mantissa: the half's value is the E4M3 value times 2^(7-15), for
// normals and subnormals alike (both formats keep subnormals).  The half -> float
// conversion is exact.  The two NaN codes (magnitude 0x7F) map to NaN.  Callers
// multiply the 2^8 back in through their per-head scale.
__device__ __forceinline__ float e4m3_to_f32_div256(uint32_t code) {
    const uint32_t mag = code & 0x7Fu;
    const uint16_t hbits = (uint16_t)(((code & 0x80u) << 8) | (mag << 7));
    const float f = (float)__builtin_bit_cast(_Float16, hbits);
    return mag == 0x7Fu ? __builtin_nanf("") : f;
}

// 8 E4M3 codes (little-endian in a uint2) -> 8 bfloat16 values (times 2^-8), exact:
// an E4M3 value has at most 4 significant bits, so truncating its float to bf16 is exact.
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8_div256(uint2 w) {
    uint4 r;
    uint32_t* o = reinterpret_cast<uint32_t*>(&r);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t word = k < 2 ? w.x : w.y;
        const int sh = (k & 1) * 16;
        const float lo = e4m3_to_f32_div256((word >> sh) & 0xFFu);
        const float hi = e4m3_to_f32_div256((word >> (sh + 8)) & 0xFFu);
        o[k] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
    return r;
}

__device__ __forceinline__ uint4 ld_global_16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ uint2 ld_global_8(const void* p) {
    return *reinterpret_cast<const uint2*>(p);
}

}  // namespace swattn
