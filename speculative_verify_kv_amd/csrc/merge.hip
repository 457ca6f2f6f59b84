// Log-sum-exp merge of split-KV partials (gfx950).
//
// Split s of a query row produced O_s (normalised over its keys) and
// lse_s = log2 of its softmax denominator in the exp2 domain.  The row's
// output is sum_s w_s O_s / sum_s w_s with w_s = 2^(lse_s - max_s lse_s); a
// split that saw no key of the row has lse_s = -inf and weight 0.  This is the
// combination step of the split-KV verify kernel named in "The Fast Gemma
// Challenge: our verified-SOTA recipe, in full" (manifest SPLITKV_VERIFY,
// "Published files"): in real arithmetic it reproduces one softmax over the
// union of the splits' keys exactly.
//
// D/4 lanes per row, each owning 4 consecutive dims (16-byte loads of every
// partial), 1024/D rows per 256-thread workgroup.  A split with no key for the
// row (lse = -inf) gets weight 2^-inf = 0, and so does every padding slot.

#include <hip/hip_runtime.h>

#include "kv_access.h"
#include "swattn_internal.h"

namespace swattn {
namespace {

template <int D, bool OUT_F32>
__global__ __launch_bounds__(kBlockThreads) void merge_kernel(MergeParams p) {
    constexpr int TPR = D / 4;
    constexpr int RPW = kBlockThreads / TPR;
    const int64_t rows_total = (int64_t)p.B * p.Hkv * p.R;
    const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / TPR;
    if (row >= rows_total) return;
    const int dq = (threadIdx.x % TPR) * 4;
    const int64_t unit = row / p.R;                 // b * Hkv + g
    const int r = (int)(row - unit * p.R);

    // Splits are taken eight at a time with every load of a chunk issued before any
    // is used; up to eight splits cost one memory round trip in all.
    constexpr int C = 8;
    const float* lse = p.ws_lse + unit * p.S * p.R + r;
    const float* o = p.ws_o + (unit * p.S * p.R + r) * D + dq;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float wsum = 0.0f;
    if (p.S <= C) {
        float l[C];
        f32x4_t v[C];
#pragma unroll
        for (int k = 0; k < C; ++k) {
            const bool in = k < p.S;
            l[k] = in ? lse[(int64_t)k * p.R] : -INFINITY;
            v[k] = in ? *reinterpret_cast<const f32x4_t*>(o + (int64_t)k * p.R * D) : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
        float M = l[0];
#pragma unroll
        for (int k = 1; k < C; ++k) M = fmaxf(M, l[k]);
        const float Mu = M == -INFINITY ? 0.0f : M;
#pragma unroll
        for (int k = 0; k < C; ++k) {
            const float w = exp2f(l[k] - Mu);
            acc += w * v[k];
            wsum += w;
        }
    } else {
        float M = -INFINITY;
        for (int s0 = 0; s0 < p.S; s0 += C) {
            float l[C];
#pragma unroll
            for (int k = 0; k < C; ++k) l[k] = s0 + k < p.S ? lse[(int64_t)(s0 + k) * p.R] : -INFINITY;
#pragma unroll
            for (int k = 0; k < C; ++k) M = fmaxf(M, l[k]);
        }
        const float Mu = M == -INFINITY ? 0.0f : M;
        for (int s0 = 0; s0 < p.S; s0 += C) {
            float l[C];
            f32x4_t v[C];
#pragma unroll
            for (int k = 0; k < C; ++k) {
                const bool in = s0 + k < p.S;
                l[k] = in ? lse[(int64_t)(s0 + k) * p.R] : -INFINITY;
                v[k] = in ? *reinterpret_cast<const f32x4_t*>(o + (int64_t)(s0 + k) * p.R * D)
                          : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
            for (int k = 0; k < C; ++k) {
                const float w = exp2f(l[k] - Mu);
                acc += w * v[k];
                wsum += w;
            }
        }
    }
    const f32x4_t res = acc * (1.0f / wsum);

    const int b = (int)(unit / p.Hkv);
    const int g = (int)(unit - (int64_t)b * p.Hkv);
    const int i = r / p.G;
    const int h = g * p.G + (r - i * p.G);
    const int64_t oi = (((int64_t)b * p.n_q + i) * p.H + h) * D + dq;
    if constexpr (OUT_F32) {
        *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.out) + oi) = res;
    } else {
        uint2 w;
        w.x = pack_bf16x2(res[0], res[1]);
        w.y = pack_bf16x2(res[2], res[3]);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + oi) = w;
    }
}

template <int D>
int launch_d(const MergeParams& p, int grid, hipStream_t st) {
    if (p.out_dtype == SWATTN_F32)
        hipLaunchKernelGGL((merge_kernel<D, true>), dim3(grid), dim3(kBlockThreads), 0, st, p);
    else
        hipLaunchKernelGGL((merge_kernel<D, false>), dim3(grid), dim3(kBlockThreads), 0, st, p);
    return (int)hipGetLastError();
}

}  // namespace

int launch_merge(const MergeParams& p, int grid, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    switch (p.D) {
        case 64: return launch_d<64>(p, grid, st);
        case 128: return launch_d<128>(p, grid, st);
        case 256: return launch_d<256>(p, grid, st);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace swattn
