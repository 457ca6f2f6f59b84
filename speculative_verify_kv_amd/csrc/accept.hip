// Greedy speculative-verify acceptance (gfx950): argmax of every position's
// logits, then the drafts accepted up to the first disagreement and the target's
// next token.
//
// Generation is greedy ("The Fast Gemma Challenge: our verified-SOTA recipe, in
// full", manifest OVERRIDE_GENERATION_CONFIG temperature 0), so the target's token
// after input i is argmax_v logits[i][v]; a verify step keeps its drafts while each
// equals the target's token before it (manifest SPECULATIVE_CONFIG), with the
// argmax fused into the step (manifest FUSED_SPARSE_ARGMAX).
//
// Argmax order: a value's float32 bits are mapped to an unsigned key that sorts as
// the values do (negative: all bits inverted; non-negative: sign bit set; -0 is
// taken as +0; every NaN maps to the largest key), and the index enters the low 32
// bits inverted, so the largest 64-bit key is the first index of the largest value.
//
// Kernel 1: one workgroup per (row, chunk of kAcceptChunk logits) reduces its chunk
// to one key in the workspace.  Kernel 2: one wave per sequence reduces the chunk
// keys of its n_q rows, writes the target ids, and scans the drafts.
//
// Inside a thread, whose logits come in increasing index order, the running maximum
// is kept as a float with its index, replaced only by a strictly larger value: the
// first index of the largest value wins and -0 equals +0, as the key order says, at
// three instructions per logit.  NaN never compares larger, so every logit is also
// added into a probe sum; a thread whose probe turns out NaN (a NaN logit, or inf and
// -inf together) scans its logits again for the first NaN.  The key is built once per
// thread from the result.

#include <hip/hip_runtime.h>

#include "swattn_internal.h"

namespace swattn {
namespace {

// 16 logits' bytes with the non-temporal cache policy: every logit is read once (64
// sequences x 8 positions x 262,144 bf16 logits: 52.2 -> 46.4 us; one sequence unchanged)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t index) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;                          // -0 -> +0
    uint32_t ord;
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        ord = 0xFFFFFFFFu;                                        // NaN
    else
        ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - index);
}

__device__ __forceinline__ uint64_t wave_max(uint64_t k) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t other = __shfl_xor(k, o, 64);
        k = other > k ? other : k;
    }
    return k;
}

// Running (maximum, index) of one thread, and the NaN probe.  The index starts at
// the thread's first logit, which is the answer when every logit is -inf.
struct ArgmaxRun {
    float best = -INFINITY;
    uint32_t idx;
    float probe = 0.0f;
    __device__ __forceinline__ explicit ArgmaxRun(uint32_t first) : idx(first) {}
    __device__ __forceinline__ void add(float v, uint32_t i) {
        const bool gt = v > best;
        best = gt ? v : best;
        idx = gt ? i : idx;
        probe += v;
    }
};

template <bool BF16>
__device__ __forceinline__ float logit_at(const void* row, int64_t v) {
    if constexpr (BF16)
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[v] << 16);
    else
        return reinterpret_cast<const float*>(row)[v];
}

template <bool BF16>
__global__ __launch_bounds__(kBlockThreads) void argmax_chunks_kernel(AcceptParams p) {
    const int nchunk = p.nchunk;
    const int64_t row = blockIdx.x / nchunk;
    const int chunk = blockIdx.x - (int)(row * nchunk);
    const int64_t v0 = (int64_t)chunk * kAcceptChunk;
    const int64_t v1 = min((int64_t)p.vocab, v0 + kAcceptChunk);
    uint64_t best = 0;                                            // below every real key
    if constexpr (BF16) {
        const uint16_t* L = reinterpret_cast<const uint16_t*>(p.logits) + row * p.vocab;
        if (p.vec_ok) {                                           // 8 logits per 16-byte load, 4 loads in flight
            constexpr int U = 4;
            const int64_t first = v0 + (int64_t)threadIdx.x * 8;
            ArgmaxRun run((uint32_t)first);
            for (int64_t v = first; v < v1; v += (int64_t)kBlockThreads * 8 * U) {
                uint4 w[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t vu = v + (int64_t)u * kBlockThreads * 8;
                    w[u] = vu < v1 ? load_stream16(L + vu) : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t vu = v + (int64_t)u * kBlockThreads * 8;
                    if (vu >= v1) break;
                    const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        run.add(__uint_as_float(ww[k] << 16), (uint32_t)(vu + 2 * k));
                        run.add(__uint_as_float(ww[k] & 0xFFFF0000u), (uint32_t)(vu + 2 * k + 1));
                    }
                }
            }
            if (run.probe != run.probe) {                         // a NaN among this thread's logits?
                for (int64_t v = first; v < v1; v += (int64_t)kBlockThreads * 8) {
                    int k = 0;
                    for (; k < 8 && v + k < v1; ++k) {
                        const float x = logit_at<true>(L, v + k);
                        if (x != x) break;
                    }
                    if (k < 8 && v + k < v1) {
                        run.best = __builtin_nanf("");
                        run.idx = (uint32_t)(v + k);
                        break;
                    }
                }
            }
            if (first < v1) best = argmax_key(run.best, run.idx);
        } else {
            for (int64_t v = v0 + threadIdx.x; v < v1; v += kBlockThreads) {
                const uint64_t a = argmax_key(__uint_as_float((uint32_t)L[v] << 16), (uint32_t)v);
                best = a > best ? a : best;
            }
        }
    } else {
        const float* L = reinterpret_cast<const float*>(p.logits) + row * p.vocab;
        if (p.vec_ok) {                                           // 4 logits per 16-byte load, 4 loads in flight
            constexpr int U = 4;
            const int64_t first = v0 + (int64_t)threadIdx.x * 4;
            ArgmaxRun run((uint32_t)first);
            for (int64_t v = first; v < v1; v += (int64_t)kBlockThreads * 4 * U) {
                float4 f[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t vu = v + (int64_t)u * kBlockThreads * 4;
                    f[u] = vu < v1 ? __builtin_bit_cast(float4, load_stream16(L + vu)) : make_float4(0, 0, 0, 0);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t vu = v + (int64_t)u * kBlockThreads * 4;
                    if (vu >= v1) break;
                    const float ff[4] = {f[u].x, f[u].y, f[u].z, f[u].w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) run.add(ff[k], (uint32_t)(vu + k));
                }
            }
            if (run.probe != run.probe) {                         // a NaN among this thread's logits?
                for (int64_t v = first; v < v1; v += (int64_t)kBlockThreads * 4) {
                    int k = 0;
                    for (; k < 4 && v + k < v1; ++k) {
                        const float x = logit_at<false>(L, v + k);
                        if (x != x) break;
                    }
                    if (k < 4 && v + k < v1) {
                        run.best = __builtin_nanf("");
                        run.idx = (uint32_t)(v + k);
                        break;
                    }
                }
            }
            if (first < v1) best = argmax_key(run.best, run.idx);
        } else {
            for (int64_t v = v0 + threadIdx.x; v < v1; v += kBlockThreads) {
                const uint64_t a = argmax_key(L[v], (uint32_t)v);
                best = a > best ? a : best;
            }
        }
    }
    __shared__ uint64_t red[kBlockThreads / 64];
    best = wave_max(best);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t k = red[0];
#pragma unroll
        for (int w = 1; w < kBlockThreads / 64; ++w) k = red[w] > k ? red[w] : k;
        p.partial[blockIdx.x] = k;
    }
}

// One wave per sequence; lane i reduces position i's chunk keys.  Every lane fetches its
// draft id up front, and the accepted count is the first lane whose draft differs from the
// target's token (a wave ballot), so no load waits on a comparison: the scan of the drafts
// one after another had made this kernel as long as the argmax pass (4.4 us).
static_assert(kAcceptMaxNq <= 64, "one lane of a wave per position");
__global__ __launch_bounds__(64) void accept_finalize_kernel(AcceptParams p) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int n_drafts = p.n_q - 1;
    const int draft = lane < n_drafts ? p.draft_ids[(int64_t)b * n_drafts + lane] : 0;
    int id = 0;
    if (lane < p.n_q) {
        const uint64_t* part = p.partial + ((int64_t)b * p.n_q + lane) * p.nchunk;
        uint64_t k = 0;
        int c = 0;
        for (; c + 8 <= p.nchunk; c += 8) {                      // eight loads in flight
            uint64_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = part[c + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) k = v[u] > k ? v[u] : k;
        }
        for (; c < p.nchunk; ++c) k = part[c] > k ? part[c] : k;
        id = (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFu));
        p.target_ids[(int64_t)b * p.n_q + lane] = id;
    }
    // draft j is accepted while it equals the target's token after input j
    const uint64_t mismatch = __ballot(lane < n_drafts && draft != id);
    const int a = mismatch != 0 ? __ffsll((unsigned long long)mismatch) - 1 : n_drafts;
    const int next = __shfl(id, a, 64);
    if (lane == 0) {
        p.accepted[b] = a;
        p.next_token[b] = next;
    }
}

}  // namespace

int launch_accept(const AcceptParams& p, int grid1, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (p.logits_dtype == SWATTN_BF16)
        hipLaunchKernelGGL((argmax_chunks_kernel<true>), dim3(grid1), dim3(kBlockThreads), 0, st, p);
    else
        hipLaunchKernelGGL((argmax_chunks_kernel<false>), dim3(grid1), dim3(kBlockThreads), 0, st, p);
    int err = (int)hipGetLastError();
    if (err != 0) return err;
    hipLaunchKernelGGL(accept_finalize_kernel, dim3(p.B), dim3(64), 0, st, p);
    return (int)hipGetLastError();
}

}  // namespace swattn
