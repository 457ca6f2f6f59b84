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

// Two floats -> packed bfloat16 bits (lo in bits 0-15), rounded as above: one two-source
// conversion (two one-source conversions and their packing cost three more instructions).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
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
// value has at most 4 significant bits and its exponent range fits bfloat16's.
// gfx950's packed conversion with scale 1.0 (v_cvt_scalef32_pk_bf16_fp8) turns two
// codes into two bfloat16s in one instruction; checked exhaustively against the
// format definition for every code in every byte position.
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 w) {
    const auto c = [](uint32_t word, bool hi) {
        return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true)
                                               : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false));
    };
    return make_uint4(c(w.x, false), c(w.x, true), c(w.y, false), c(w.y, true));
}

__device__ __forceinline__ uint4 ld_global_16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ uint2 ld_global_8(const void* p) {
    return *reinterpret_cast<const uint2*>(p);
}

}  // namespace swattn
