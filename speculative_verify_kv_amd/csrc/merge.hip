// Log-sum-exp merge of split-KV partials (gfx950): the separate merge kernel, for
// launches whose partition workgroups do not combine their partials themselves.
// The combination (split_merge.h) is the step of the split-KV verify kernel named
// in "The Fast Gemma Challenge: our verified-SOTA recipe, in full" (manifest
// SPLITKV_VERIFY, "Published files").
//
// D/4 lanes per row, each owning 4 consecutive dims (16-byte loads of every
// partial), 4 kMergeThreads / D rows per workgroup.

#include <hip/hip_runtime.h>

#include "kv_access.h"
#include "split_merge.h"
#include "swattn_internal.h"

namespace swattn {
namespace {

template <int D, bool OUT_F32>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams p) {
    constexpr int TPR = D / 4;
    constexpr int RPW = kMergeThreads / TPR;
    const int64_t rows_total = (int64_t)p.B * p.Hkv * p.R;
    const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / TPR;
    if (row >= rows_total) return;
    const int dq = (threadIdx.x % TPR) * 4;
    const int64_t unit = row / p.R;                 // b * Hkv + g
    const int r = (int)(row - unit * p.R);

    const f32x4_t res = combine_splits4<D>(p.ws_o, p.ws_lse, unit, p.S, p.R, r, dq);

    const int b = (int)(unit / p.Hkv);
    const int g = (int)(unit - (int64_t)b * p.Hkv);
    const int i = r / p.G;
    const int h = g * p.G + (r - i * p.G);
    const int64_t oi = (((int64_t)b * p.n_q + i) * p.H + h) * D + dq;
    store_out4<OUT_F32>(p.out, oi, res);
}

template <int D>
int launch_d(const MergeParams& p, int grid, hipStream_t st) {
    if (p.out_dtype == SWATTN_F32)
        hipLaunchKernelGGL((merge_kernel<D, true>), dim3(grid), dim3(kMergeThreads), 0, st, p);
    else
        hipLaunchKernelGGL((merge_kernel<D, false>), dim3(grid), dim3(kMergeThreads), 0, st, p);
    return (int)hipGetLastError();
}

}  // namespace

// Zero fill of the workspace's arrival counters (a kernel, not a memset node, so
// that it can sit in a captured graph).
__global__ __launch_bounds__(kBlockThreads) void zero_words_kernel(int32_t* w, int n) {
    const int i = blockIdx.x * kBlockThreads + threadIdx.x;
    if (i < n) w[i] = 0;
}

int launch_zero_words(int32_t* w, int n, void* stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(zero_words_kernel, dim3((n + kBlockThreads - 1) / kBlockThreads), dim3(kBlockThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), w, n);
    return (int)hipGetLastError();
}

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
