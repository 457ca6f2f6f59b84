// Log-sum-exp combination of split-KV partials (gfx950), shared by the merge
// kernel and the partition kernels' fused tail.
//
// Split s of a query row produced O_s (normalised over its keys) and lse_s = log2
// of its softmax denominator in the exp2 domain.  The row's output is
// sum_s w_s O_s / sum_s w_s with w_s = 2^(lse_s - max_s lse_s); a split that saw
// no key of the row has lse_s = -inf and weight 0.  In real arithmetic this is one
// softmax over the union of the splits' keys, the combination step of the
// split-KV verify kernel named in "The Fast Gemma Challenge: our verified-SOTA
// recipe, in full" (manifest SPLITKV_VERIFY, "Published files").
//
// Workspace rows: partial (unit, s, r) sits at ((unit * S + s) * R + r), unit =
// b * Hkv + g; ws_o holds D floats per row, ws_lse one.
#pragma once

#include <hip/hip_runtime.h>

#include "kv_access.h"
#include "swattn_internal.h"

namespace swattn {

// Device-coherent accesses for partials that another workgroup of the same launch
// reads (it may run on another XCD, whose L2 is not this one's): loads and stores
// with the sc1 cache-policy bit, which on gfx950 makes them go past the XCD's L2 to
// the device-coherent level (the bit the compiler sets for agent-scope atomics).
// Written as inline assembly so that 16-byte accesses keep it; the compiler does not
// track these, so every use of a loaded value follows an explicit vmcnt wait
// (coherent_wait) and the stores are waited for in merge_if_last.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void store_coherent4(float* p, f32x4_t v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_coherent1(float* p, float v) {
    asm volatile("global_store_dword %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ f32x4_t load_coherent4(const float* p) {
    f32x4_t v;
    asm volatile("global_load_dwordx4 %0, %1, off sc1" : "=v"(v) : "v"(p) : "memory");
    return v;
}
__device__ __forceinline__ float load_coherent1(const float* p) {
    float v;
    asm volatile("global_load_dword %0, %1, off sc1" : "=v"(v) : "v"(p) : "memory");
    return v;
}
#pragma clang diagnostic pop
// Waits for every coherent load issued so far; the empty asm statements after it pin
// the uses of the loaded registers behind the wait.
template <int C>
__device__ __forceinline__ void coherent_wait(float (&l)[C], f32x4_t (&v)[C]) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int k = 0; k < C; ++k) asm volatile("" : "+v"(l[k]), "+v"(v[k]));
}

// A partition workgroup's partial: plain stores when a merge kernel reads them after
// the launch, device-coherent stores when the launch's last workgroup does.
__device__ __forceinline__ void store_partial4(const PartitionParams& p, float* dst, f32x4_t v) {
    if (p.counters != nullptr)
        store_coherent4(dst, v);
    else
        *reinterpret_cast<f32x4_t*>(dst) = v;
}
__device__ __forceinline__ void store_partial1(const PartitionParams& p, float* dst, float v) {
    if (p.counters != nullptr)
        store_coherent1(dst, v);
    else
        *dst = v;
}

// Splits s0 .. s0+C-1 of one row's partials (lse, 4 dims): plain loads, or coherent
// loads followed by their wait.  Slots past S get lse -inf (weight 0) and zeros.
template <int D, int C, bool COHERENT>
__device__ __forceinline__ void load_split_group(const float* lse, const float* o, int S, int R, int s0,
                                                 float (&l)[C], f32x4_t (&v)[C]) {
#pragma unroll
    for (int k = 0; k < C; ++k) {
        const bool in = s0 + k < S;
        const int64_t sk = s0 + k;
        if constexpr (COHERENT) {
            l[k] = -INFINITY;
            v[k] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            if (in) {
                l[k] = load_coherent1(lse + sk * R);
                v[k] = load_coherent4(o + sk * R * D);
            }
        } else {
            l[k] = in ? lse[sk * R] : -INFINITY;
            v[k] = in ? *reinterpret_cast<const f32x4_t*>(o + sk * R * D) : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
    if constexpr (COHERENT) coherent_wait<C>(l, v);
}

// Dims dq .. dq+3 of row r of `unit`, combined over the S splits.  Splits are taken
// eight at a time with every load of a group issued before any is used.
template <int D, bool COHERENT = false>
__device__ __forceinline__ f32x4_t combine_splits4(const float* ws_o, const float* ws_lse, int64_t unit,
                                                   int S, int R, int r, int dq) {
    constexpr int C = 8;
    const float* lse = ws_lse + unit * S * R + r;
    const float* o = ws_o + (unit * S * R + r) * D + dq;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float wsum = 0.0f;
    float l[C];
    f32x4_t v[C];
    if (S <= C) {
        load_split_group<D, C, COHERENT>(lse, o, S, R, 0, l, v);
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
        for (int s0 = 0; s0 < S; s0 += C) {
            load_split_group<D, C, COHERENT>(lse, o, S, R, s0, l, v);
#pragma unroll
            for (int k = 0; k < C; ++k) M = fmaxf(M, l[k]);
        }
        const float Mu = M == -INFINITY ? 0.0f : M;
        for (int s0 = 0; s0 < S; s0 += C) {
            load_split_group<D, C, COHERENT>(lse, o, S, R, s0, l, v);
#pragma unroll
            for (int k = 0; k < C; ++k) {
                const float w = exp2f(l[k] - Mu);
                acc += w * v[k];
                wsum += w;
            }
        }
    }
    return acc * (1.0f / wsum);
}

// Four consecutive output values at element offset oi.
template <bool OUT_F32>
__device__ __forceinline__ void store_out4(void* out, int64_t oi, f32x4_t v) {
    if constexpr (OUT_F32) {
        *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + oi) = v;
    } else {
        uint2 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + oi) = w;
    }
}

// Fused tail of a partition workgroup that wrote its split's partials: the last of
// the S workgroups of a merge group combines the group's partials and writes the
// output, so no merge kernel runs.  A merge group is one (problem, KV head, row
// chunk, column split): its S workgroups wrote the partials of the chunk's rows and
// the split's output columns cs * D/col_splits .. +D/col_splits, one key split
// each, and the workgroup that counts last combines exactly those columns.
//
// Arrival is counted in p.counters[((b * Hkv + g) * row_chunks + rc) * col_splits
// + cs], which must be zero when the call starts; the last of the group's S
// workgroups sets it back to zero.  The partials were written with
// device-coherent stores (store_partial4/1); every wave waits until its stores have
// completed before the workgroup counts itself (an agent-scope atomic add), and the
// workgroup that counts last reads the partials with device-coherent loads, issued
// only after its count returned.  (A device-scope release fence would also do, but
// on gfx950 it writes back the XCD's whole L2, once per wave: tens of microseconds
// per launch.)  Every thread of every workgroup must call this: it contains
// barriers.
//
// Why this ordering suffices: the LLVM AMDGPU memory model (AMDGPUUsage, "Memory
// Model GFX942", which gfx950 follows) implements an agent-scope release as "wait
// for every earlier store to complete" (s_waitcnt vmcnt(0)) plus a write-back of the
// L2 lines that other agents' caches may not see, and an agent-scope acquire as an
// invalidate of the L1 / non-coherent L2 lines before later loads.  Here the only
// data that crosses workgroups is written with sc1 stores, which go past the
// non-coherent L2 to the device-coherent level, and read with sc1 loads, which miss
// in the non-coherent caches; so the wait for the stores is the whole release and
// the coherent loads after the atomic's return are the whole acquire.  The atomic
// itself is relaxed: the waits before it (stores complete, then a barrier) and the
// control dependency after it (loads are issued only once its value returned and
// the barrier published it) order the accesses.
template <int D, bool OUT_F32, int NT>
__device__ __forceinline__ void merge_if_last(const PartitionParams& p, int b, int g, int rc, int cs) {
    __shared__ int last;
    __builtin_amdgcn_s_waitcnt(0);           // this wave's partial stores are done
    __syncthreads();
    if (threadIdx.x == 0) {
        int* c = p.counters + (((int64_t)b * p.Hkv + g) * p.row_chunks + rc) * p.col_splits + cs;
        const int arrived = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
        const bool is_last = arrived == p.S;
        // every split has counted: ready for the next call
        if (is_last) __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = is_last;
    }
    __syncthreads();
    if (!last) return;
    const int DC = D / p.col_splits;             // the group's output columns
    const int TPR = DC / 4;                      // threads per row, 4 dims each
    const int64_t unit = (int64_t)b * p.Hkv + g;
    const int r0 = rc * p.rows_per_chunk;
    const int nr = min(p.R - r0, p.rows_per_chunk);
    for (int slot = threadIdx.x; slot < nr * TPR; slot += NT) {
        const int r = r0 + slot / TPR;
        const int dq = cs * DC + (slot % TPR) * 4;
        const f32x4_t v = combine_splits4<D, true>(p.ws_o, p.ws_lse, unit, p.S, p.R, r, dq);
        const int i = r / p.G;
        const int h = g * p.G + (r - i * p.G);
        store_out4<OUT_F32>(p.out, (((int64_t)b * p.n_q + i) * p.H + h) * D + dq, v);
    }
}

}  // namespace swattn
