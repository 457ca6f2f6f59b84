// Split-KV partition kernel on the vector ALUs, fp32 arithmetic (gfx950).
//
// Used when Q or the cache is float32, where a bf16 matrix-core tile would lose
// precision (and whenever the caller asks for it).  One workgroup owns one
// (problem b, KV head g, 8-row chunk, KV split s) and at most 256 keys:
//
//   phase 0  the cache row of every key of the split, from the block table, into
//            LDS (one pass, every key in parallel);
//   phase 1  scores: 4 lanes per key, each dotting a quarter of the head
//            dimension against the 8 rows held in LDS, two xor-shuffles to sum;
//            the window mask (t - W, t] is applied here, scores kept in LDS;
//   phase 2  exact softmax per row (one wave per row, max and sum by shuffles);
//   phase 3  P V: each lane owns 4 consecutive dims of every row and a strided
//            subset of the keys (coalesced V rows), partial sums meet in LDS.
//
// The kernel is a chain of dependent memory round trips, so phases 1 and 3 issue
// the loads of several rounds (keys) before using any of them: one batch of loads
// in flight per round trip instead of one round's.
//
// The result is the final output (S == 1) or a normalised partial plus its
// log2-sum-exp for the merge kernel (S > 1).  Semantics: "The Fast Gemma
// Challenge: our verified-SOTA recipe, in full" (manifest SLIDING_WINDOW,
// SPECULATIVE_CONFIG, SPLITKV_VERIFY; "What each piece does, and why").

#include <hip/hip_runtime.h>

#include "kv_access.h"
#include "split_merge.h"
#include "swattn_internal.h"

namespace swattn {
namespace {

enum { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

// N consecutive cached elements starting at element offset `off` -> float.
template <int KVT, int N>
__device__ __forceinline__ void load_kv(const void* base, int64_t off, float* dst) {
    if constexpr (KVT == KV_F32) {
        const float* src = reinterpret_cast<const float*>(base) + off;
#pragma unroll
        for (int k = 0; k < N; k += 4) {
            const float4 v = *reinterpret_cast<const float4*>(src + k);
            dst[k] = v.x; dst[k + 1] = v.y; dst[k + 2] = v.z; dst[k + 3] = v.w;
        }
    } else if constexpr (KVT == KV_BF16) {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(base) + off;
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int k = 0; k < N; k += 8) {
                const uint4 v = ld_global_16(src + k);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dst[k + 2 * e] = bf16_bits_to_f32(w[e] & 0xFFFFu);
                    dst[k + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                }
            }
        } else {
            static_assert(N == 4, "bf16 loads of 4 or a multiple of 8");
            const uint2 v = ld_global_8(src);
            dst[0] = bf16_bits_to_f32(v.x & 0xFFFFu);
            dst[1] = __uint_as_float(v.x & 0xFFFF0000u);
            dst[2] = bf16_bits_to_f32(v.y & 0xFFFFu);
            dst[3] = __uint_as_float(v.y & 0xFFFF0000u);
        }
    } else {
        const uint8_t* src = reinterpret_cast<const uint8_t*>(base) + off;
        if constexpr (N % 16 == 0) {
#pragma unroll
            for (int k = 0; k < N; k += 16) {
                const uint4 v = ld_global_16(src + k);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 16; e += 2) e4m3x2_to_f32(w[e >> 2], (e & 2) != 0, dst[k + e], dst[k + e + 1]);
            }
        } else {
            static_assert(N == 4, "e4m3 loads of 4 or a multiple of 16");
            const uint32_t w = *reinterpret_cast<const uint32_t*>(src);
            e4m3x2_to_f32(w, false, dst[0], dst[1]);
            e4m3x2_to_f32(w, true, dst[2], dst[3]);
        }
    }
}

// Element offset of key j's cache row for KV head g, or -1 for a block id outside the pool.
__device__ __forceinline__ int64_t valu_row_offset(const PartitionParams& p, int b, int g, int j) {
    const int blk = j / p.bs;
    const int off = j - blk * p.bs;
    const int phys = p.block_table[(int64_t)b * p.max_blocks + blk];
    if (phys < 0 || phys >= p.num_blocks) return -1;
    return (((int64_t)phys * p.Hkv + g) * p.bs + off) * (int64_t)p.D;
}

// Lane exchanges without the LDS crossbar (__shfl_xor goes through ds_bpermute, one
// round trip through the LDS per step, which made the softmax of a handful of rows take
// 1.3 us): DPP moves within each 16-lane row, then gfx950's lane-group swaps across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;    // quad_perm [1, 0, 3, 2]: lane l reads lane l ^ 1
constexpr int kDppXor2 = 0x4E;    // quad_perm [2, 3, 0, 1]: lane l reads lane l ^ 2
constexpr int kDppRor4 = 0x124;   // row_ror:4 within the 16-lane row
constexpr int kDppRor8 = 0x128;   // row_ror:8

// Sum over the 4 lanes of a quad (l & ~3 .. l | 3), every lane receiving it.
__device__ __forceinline__ float quad_sum(float x) {
    x += dpp_mov<kDppXor1>(x);
    return x + dpp_mov<kDppXor2>(x);
}

// Max / sum over all 64 lanes of the wave, every lane receiving the result.
template <bool MAX>
__device__ __forceinline__ float wave_reduce(float x) {
    const auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    x = op(x, dpp_mov<kDppXor1>(x));
    x = op(x, dpp_mov<kDppXor2>(x));
    x = op(x, dpp_mov<kDppRor4>(x));   // each lane: its quad and the next
    x = op(x, dpp_mov<kDppRor8>(x));   // the whole 16-lane row
    // rows l, l ^ 16, l ^ 32, l ^ 48: each swap returns the value and its partner's
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return op(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

template <int D, int KVT>
__global__ __launch_bounds__(kBlockThreads) void partition_valu_kernel(PartitionParams p) {
    constexpr int RC = kValuRowsPerChunk;
    constexpr int KR = kValuKeyRound;
    constexpr int TPK = kBlockThreads / KR;   // 4 lanes per key in phase 1
    static_assert(TPK == 4, "a key's lanes are one quad (quad_sum)");
    constexpr int DPT = D / TPK;              // dims per lane in phase 1
    constexpr int QPR = D / 4;                // phase-3 lanes per row
    constexpr int KGR = kBlockThreads / QPR;  // phase-3 key groups
    constexpr int RPB = D >= 128 ? 2 : 4;     // phase-1 rounds whose loads go out together
    constexpr int U3 = 8;                     // phase-3 keys per lane whose loads go out together

    __shared__ float qs[RC][D];
    __shared__ float ps[RC][kValuMaxKeys];
    __shared__ __attribute__((aligned(16))) float red[KGR][RC][D];
    __shared__ float rstat[RC][2];
    __shared__ int64_t roff[kValuMaxKeys];    // cache row of key k0 + kk (element offset), or -1
    __shared__ int tbl[kBlockThreads];        // the problem's block-table row, when it is that short

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    int lin = blockIdx.x;
    const int s = lin % p.S;
    lin /= p.S;
    const int rc = lin % p.row_chunks;
    lin /= p.row_chunks;
    const int g = lin % p.Hkv;
    const int b = lin / p.Hkv;

    // A block-table row that fits one entry per thread is read while ctx_len is in
    // flight: one dependent round trip fewer before the first K loads.
    const bool short_row = p.max_blocks <= kBlockThreads;
    const int tb = (short_row && tid < p.max_blocks) ? p.block_table[(int64_t)b * p.max_blocks + tid] : 0;
    const int ctx = p.ctx_len[b];
    const bool seq_ok = ctx >= p.n_q && ctx <= p.max_blocks * p.bs && ctx <= p.max_ctx;
    const int pos0 = seq_ok ? ctx - p.n_q : 0;
    // the chunk's keys: the union of its rows' windows (queries qi_lo .. qi_hi)
    const int qi_lo = rc * p.rows_per_chunk / p.G;
    const int qi_hi = min(p.R - 1, rc * p.rows_per_chunk + p.rows_per_chunk - 1) / p.G;
    const int u_lo = max(0, pos0 + qi_lo - p.window + 1);
    const int u_hi = pos0 + qi_hi + 1;                   // one past the last key
    int k0 = 0, nk = 0;
    if (seq_ok) {
        const int kps = (u_hi - u_lo + p.S - 1) / p.S;
        k0 = u_lo + s * kps;
        nk = max(0, min(u_hi, k0 + kps) - k0);
    }

    float sl2 = p.scale_log2;
    float osc = 1.0f;
    if constexpr (KVT == KV_FP8) {
        sl2 *= p.k_scale[g];
        osc = p.v_scale[g];
    }

    // ---- Q rows of this chunk -> LDS (float) ---------------------------------------
    for (int idx = tid; idx < RC * D; idx += kBlockThreads) {
        const int rr = idx / D, d = idx - rr * D;
        const int r = rc * RC + rr;
        float val = 0.0f;
        if (r < p.R) {
            const int i = r / p.G;
            const int h = g * p.G + (r - i * p.G);
            const int64_t qi = (((int64_t)b * p.n_q + i) * p.H + h) * D + d;
            val = p.q_dtype == SWATTN_F32 ? reinterpret_cast<const float*>(p.q)[qi]
                                          : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.q)[qi]);
        }
        qs[rr][d] = val;
    }
    if (short_row) tbl[tid] = tb;
    __syncthreads();

    // ---- phase 0: cache rows of the split's keys -> LDS --------------------------------
    for (int kk = tid; kk < nk; kk += kBlockThreads) {
        const int j = k0 + kk;
        if (short_row) {
            const int blk = j / p.bs;
            const int phys = tbl[blk];
            roff[kk] = (phys < 0 || phys >= p.num_blocks) ? -1
                                                          : (((int64_t)phys * p.Hkv + g) * p.bs + (j - blk * p.bs)) * (int64_t)p.D;
        } else {
            roff[kk] = valu_row_offset(p, b, g, j);
        }
    }
    __syncthreads();

    // ---- phase 1: masked scores (log2 domain) ------------------------------------------
    {
        const int slot = tid / TPK;
        const int part = tid % TPK;
        for (int kb = 0; kb < nk; kb += RPB * KR) {
        float kvb[RPB][DPT];
#pragma unroll
        for (int u = 0; u < RPB; ++u) {
            const int kk = kb + u * KR + slot;
            if (kk < nk) {
                const int64_t off = roff[kk];
                if (off >= 0) {
                    load_kv<KVT, DPT>(p.k, off + part * DPT, kvb[u]);
                } else {
#pragma unroll
                    for (int e = 0; e < DPT; ++e) kvb[u][e] = __builtin_nanf("");
                }
            } else {
#pragma unroll
                for (int e = 0; e < DPT; ++e) kvb[u][e] = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < RPB; ++u) {
            const int kk = kb + u * KR + slot;
            if (kb + u * KR >= nk) break;
            const bool valid = kk < nk;
            const int j = k0 + kk;
            const float* kv = kvb[u];
            float dots[RC];
#pragma unroll
            for (int rr = 0; rr < RC; ++rr) {
                float acc = 0.0f;
#pragma unroll
                for (int e = 0; e < DPT; ++e) acc = fmaf(qs[rr][part * DPT + e], kv[e], acc);
                dots[rr] = quad_sum(acc);
            }
            if (part == 0 && valid) {
#pragma unroll
                for (int rr = 0; rr < RC; ++rr) {
                    const int r = rc * RC + rr;
                    const int i = r / p.G;
                    const int lo = max(0, pos0 + i - p.window + 1);
                    const int hi = pos0 + i;
                    const bool ok = r < p.R && j >= lo && j <= hi;
                    ps[rr][kk] = ok ? dots[rr] * sl2 : -INFINITY;
                }
            }
        }
        }
    }
    __syncthreads();

    // ---- phase 2: exact softmax of each row over this split's keys ---------------------
    for (int rr = wave; rr < RC; rr += kBlockThreads / kWaveSize) {
        float m = -INFINITY;
        for (int kk = lane; kk < nk; kk += kWaveSize) m = fmaxf(m, ps[rr][kk]);
        m = wave_reduce<true>(m);
        const float mu = m == -INFINITY ? 0.0f : m;
        float sum = 0.0f;
        for (int kk = lane; kk < nk; kk += kWaveSize) {
            const float e = exp2f(ps[rr][kk] - mu);
            ps[rr][kk] = e;
            sum += e;
        }
        sum = wave_reduce<false>(sum);
        if (lane == 0) {
            rstat[rr][0] = m;
            rstat[rr][1] = sum;
        }
    }
    __syncthreads();

    // ---- phase 3: P V ------------------------------------------------------------------
    {
        const int dq = (tid % QPR) * 4;
        const int kgp = tid / QPR;
        float acc[RC][4];
#pragma unroll
        for (int rr = 0; rr < RC; ++rr) acc[rr][0] = acc[rr][1] = acc[rr][2] = acc[rr][3] = 0.0f;
        for (int kb = kgp; kb < nk; kb += U3 * KGR) {
            float vb[U3][4];
#pragma unroll
            for (int u = 0; u < U3; ++u) {
                const int kk = kb + u * KGR;
                vb[u][0] = vb[u][1] = vb[u][2] = vb[u][3] = 0.0f;
                if (kk < nk) {
                    const int64_t off = roff[kk];
                    if (off >= 0) {
                        load_kv<KVT, 4>(p.v, off + dq, vb[u]);
                    } else {
                        vb[u][0] = vb[u][1] = vb[u][2] = vb[u][3] = __builtin_nanf("");
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U3; ++u) {
                const int kk = kb + u * KGR;
                if (kk >= nk) break;
#pragma unroll
                for (int rr = 0; rr < RC; ++rr) {
                    const float pr = ps[rr][kk];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[rr][e] = fmaf(pr, vb[u][e], acc[rr][e]);
                }
            }
        }
#pragma unroll
        for (int rr = 0; rr < RC; ++rr)
            *reinterpret_cast<float4*>(&red[kgp][rr][dq]) = make_float4(acc[rr][0], acc[rr][1], acc[rr][2], acc[rr][3]);
    }
    __syncthreads();

    const float poison = seq_ok ? 0.0f : __builtin_nanf("");
    for (int idx = tid; idx < RC * D; idx += kBlockThreads) {
        const int rr = idx / D, d = idx - rr * D;
        const int r = rc * RC + rr;
        if (r >= p.R) continue;
        float sum = 0.0f;
#pragma unroll
        for (int k = 0; k < KGR; ++k) sum += red[k][rr][d];
        const float L = rstat[rr][1];
        // L == 0: no key of this split is in the row's window.  A NaN L (NaN read from
        // the cache or an out-of-range block) must reach the output, so test == 0.
        const float val = (L == 0.0f ? 0.0f : sum * (osc / L)) + poison;
        if (p.S == 1) {
            const int i = r / p.G;
            const int h = g * p.G + (r - i * p.G);
            const int64_t oi = (((int64_t)b * p.n_q + i) * p.H + h) * D + d;
            if (p.out_dtype == SWATTN_F32)
                reinterpret_cast<float*>(p.out)[oi] = val;
            else
                reinterpret_cast<uint16_t*>(p.out)[oi] = (uint16_t)f32_to_bf16_bits(val);
        } else {
            const int64_t prow = (((int64_t)b * p.Hkv + g) * p.S + s) * p.R + r;
            store_partial1(p, p.ws_o + prow * D + d, val);
            if (d == 0)
                store_partial1(p, p.ws_lse + prow, (L == 0.0f ? -INFINITY : rstat[rr][0] + log2f(L)) + poison);
        }
    }
    // split launches: the last workgroup of the row chunk combines the partials (one
    // column split: the group is the whole chunk)
    if (p.counters != nullptr) {
        if (p.out_dtype == SWATTN_F32)
            merge_if_last<D, true, kBlockThreads>(p, b, g, rc, 0);
        else
            merge_if_last<D, false, kBlockThreads>(p, b, g, rc, 0);
    }
}

template <int D>
int launch_d(const PartitionParams& p, int grid, hipStream_t st) {
    switch (p.kv_dtype) {
        case SWATTN_F32:
            hipLaunchKernelGGL((partition_valu_kernel<D, KV_F32>), dim3(grid), dim3(kBlockThreads), 0, st, p);
            break;
        case SWATTN_BF16:
            hipLaunchKernelGGL((partition_valu_kernel<D, KV_BF16>), dim3(grid), dim3(kBlockThreads), 0, st, p);
            break;
        default:
            hipLaunchKernelGGL((partition_valu_kernel<D, KV_FP8>), dim3(grid), dim3(kBlockThreads), 0, st, p);
            break;
    }
    return (int)hipGetLastError();
}

}  // namespace

int launch_partition_valu(const PartitionParams& p, int grid, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    switch (p.D) {
        case 64: return launch_d<64>(p, grid, st);
        case 128: return launch_d<128>(p, grid, st);
        case 256: return launch_d<256>(p, grid, st);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace swattn
