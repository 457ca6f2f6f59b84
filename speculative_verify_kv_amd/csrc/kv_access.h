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

// OCP E4M3 -> float, exactly, with gfx950's conversion instruction
// (v_cvt_pk_f32_fp8 decodes the OCP E4M3 format on this target: bias 7,
// subnormals kept, S.1111.111 is NaN).  `hi` selects bytes 2-3 instead of 0-1.
__device__ __forceinline__ void e4m3x2_to_f32(uint32_t word, bool hi, float& a, float& b) {
    const auto v = hi ? __builtin_amdgcn_cvt_pk_f32_fp8(word, true) : __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
    a = v[0];
    b = v[1];
}

// 8 E4M3 codes (little-endian in a uint2) -> 8 bfloat16 values, exactly: an E4M3
// value has at most 4 significant bits, so keeping the upper half of its float is exact.
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 w) {
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float a, b;
        e4m3x2_to_f32(k < 2 ? w.x : w.y, (k & 1) != 0, a, b);
        o[k] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ uint4 ld_global_16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ uint2 ld_global_8(const void* p) {
    return *reinterpret_cast<const uint2*>(p);
}

}  // namespace swattn
