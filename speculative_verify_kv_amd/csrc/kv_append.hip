// KV-cache append: the n_new K and V rows of every sequence go into the paged
// cache, converted to the cache's element type (gfx950).
//
// A verify step scores the target token and its drafts ("The Fast Gemma
// Challenge: our verified-SOTA recipe, in full", manifest SPECULATIVE_CONFIG),
// so their K/V rows must be in the cache before the attention call reads them.
// Row (b, i, g) goes to position t = ctx_len[b] - n_new + i: block
// block_table[b][t / bs], offset t % bs.  A sequence whose ctx_len is outside its
// valid range, or a position whose block id is outside the pool, is skipped: the
// kernel never writes where it should not.
//
// Conversions: bfloat16 rounds to nearest even; E4M3 takes the float32 quotient
// by the head's scale (correctly rounded division) and rounds it to the nearest
// E4M3 value, ties to the even code, saturating at 448 (no infinities in E4M3),
// NaN to the NaN code with its sign.  The rounding is done on the quotient's bits
// from the format definition (1 sign, 4 exponent bits with bias 7, 3 mantissa
// bits; exponent 0 holds the subnormals m * 2^-9).
//
// One thread moves 8 elements of one row: 16 or 32 bytes in, 8 to 32 bytes out.

#include <hip/hip_runtime.h>

#include "kv_access.h"
#include "swattn_internal.h"

namespace swattn {
namespace {

// float32 -> E4M3 code, round to nearest even, saturating (see the file comment).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float q) {
    const uint32_t u = __float_as_uint(q);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return sign | 0x7Fu;                 // NaN
    if (a >= 0x43E00000u) return sign | 0x7Eu;                // |q| >= 448, infinities included
    if (a < 0x3C800000u) {                                    // |q| < 2^-6: subnormal step 2^-9
        // |q| * 2^9 < 8 is exact; rintf rounds it to the nearest integer, ties to even;
        // 8 is the smallest normal's code
        return sign | (uint32_t)rintf(__uint_as_float(a) * 512.0f);
    }
    const uint32_t e = (a >> 23) - 127u + 7u;                 // biased E4M3 exponent, 1 .. 15
    const uint32_t m3 = (a >> 20) & 7u;                       // top three mantissa bits
    const uint32_t rest = a & 0xFFFFFu;                       // the 20 dropped bits
    uint32_t code = (e << 3) | m3;
    if (rest > 0x80000u || (rest == 0x80000u && (m3 & 1u))) code += 1u;   // may carry into the exponent
    return sign | code;                                       // below 448 it stays <= 0x7E
}

template <int NEW, int KV>   // NEW: SWATTN_F32 / SWATTN_BF16; KV: SWATTN_F32 / SWATTN_BF16 / SWATTN_FP8_E4M3
__global__ __launch_bounds__(kBlockThreads) void kv_append_kernel(AppendParams p) {
    const int cpr = p.D / 8;                                  // 8-element chunks per row
    const int64_t per_tensor = (int64_t)p.B * p.n_new * p.Hkv * cpr;
    const int64_t idx = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
    if (idx >= 2 * per_tensor) return;
    const bool is_v = idx >= per_tensor;
    int64_t r = is_v ? idx - per_tensor : idx;
    const int c = (int)(r % cpr);
    r /= cpr;
    const int g = (int)(r % p.Hkv);
    r /= p.Hkv;
    const int i = (int)(r % p.n_new);
    const int b = (int)(r / p.n_new);

    const int ctx = p.ctx_len[b];
    if (ctx < p.n_new || ctx > p.max_blocks * p.bs || ctx > p.max_ctx) return;
    const int t = ctx - p.n_new + i;
    const int blk = t / p.bs;
    const int phys = p.block_table[(int64_t)b * p.max_blocks + blk];
    if (phys < 0 || phys >= p.num_blocks) return;
    const int64_t dst = (((int64_t)phys * p.Hkv + g) * p.bs + (t - blk * p.bs)) * p.D + c * 8;
    const int64_t src = (((int64_t)b * p.n_new + i) * p.Hkv + g) * p.D + c * 8;

    // 8 source values as float32
    float x[8];
    if constexpr (NEW == SWATTN_F32) {
        const float* s = reinterpret_cast<const float*>(is_v ? p.v_new : p.k_new) + src;
        const float4 a = *reinterpret_cast<const float4*>(s);
        const float4 bq = *reinterpret_cast<const float4*>(s + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = bq.x; x[5] = bq.y; x[6] = bq.z; x[7] = bq.w;
    } else {
        const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(is_v ? p.v_new : p.k_new) + src);
        if constexpr (KV == SWATTN_BF16) {               // bfloat16 -> bfloat16: a plain copy
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(is_v ? p.v_cache : p.k_cache) + dst) = w;
            return;
        }
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = __uint_as_float(ww[k] << 16);
            x[2 * k + 1] = __uint_as_float(ww[k] & 0xFFFF0000u);
        }
    }

    if constexpr (KV == SWATTN_F32) {
        float* d = reinterpret_cast<float*>(is_v ? p.v_cache : p.k_cache) + dst;
        *reinterpret_cast<float4*>(d) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4*>(d + 4) = make_float4(x[4], x[5], x[6], x[7]);
    } else if constexpr (KV == SWATTN_BF16) {
        uint4 o;
        o.x = pack_bf16x2(x[0], x[1]);
        o.y = pack_bf16x2(x[2], x[3]);
        o.z = pack_bf16x2(x[4], x[5]);
        o.w = pack_bf16x2(x[6], x[7]);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(is_v ? p.v_cache : p.k_cache) + dst) = o;
    } else {
        const float s = (is_v ? p.v_scale : p.k_scale)[g];
        uint32_t code[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) code[k] = e4m3_rne_sat(x[k] / s);
        uint2 o;
        o.x = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
        o.y = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(is_v ? p.v_cache : p.k_cache) + dst) = o;
    }
}

template <int NEW>
int launch_new(const AppendParams& p, int grid, hipStream_t st) {
    switch (p.kv_dtype) {
        case SWATTN_F32:
            hipLaunchKernelGGL((kv_append_kernel<NEW, SWATTN_F32>), dim3(grid), dim3(kBlockThreads), 0, st, p);
            break;
        case SWATTN_BF16:
            hipLaunchKernelGGL((kv_append_kernel<NEW, SWATTN_BF16>), dim3(grid), dim3(kBlockThreads), 0, st, p);
            break;
        case SWATTN_FP8_E4M3:
            hipLaunchKernelGGL((kv_append_kernel<NEW, SWATTN_FP8_E4M3>), dim3(grid), dim3(kBlockThreads), 0, st, p);
            break;
        default:
            return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

}  // namespace

int launch_kv_append(const AppendParams& p, int grid, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (p.new_dtype == SWATTN_F32) return launch_new<SWATTN_F32>(p, grid, st);
    if (p.new_dtype == SWATTN_BF16) return launch_new<SWATTN_BF16>(p, grid, st);
    return (int)hipErrorInvalidValue;
}

}  // namespace swattn
