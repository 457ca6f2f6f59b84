// swattn_window_gather: the data movement of a verify call without its arithmetic, as a
// measurement of the floor that the paged layout and the launch shape set; and
// swattn_stream_read: a contiguous read of a given size, the floor that HBM sets.
//
// `parts` workgroups per (problem b, KV head g) move exactly the bytes the verify
// call's algorithmic count covers: the K and V rows of the union of its queries'
// windows (positions ctx_len[b] - n_q - window + 1 .. ctx_len[b] - 1, clipped at 0),
// read through the block table with the same 16-byte global-to-LDS loads as the
// partition kernel, all requested at once; its Q rows, the same way; and an
// output-sized write of zeros.  Workgroup p of a unit takes the p-th contiguous slice
// of each (window rows, Q rows, output rows).  Nothing is computed.  The loaded bytes
// land in one LDS buffer that is overwritten freely; every load is waited for before
// the workgroup ends.  A window of more than 1024 rows is measured over its first 1024
// (and at most 512 Q rows).
//
// The window rule follows "The Fast Gemma Challenge: our verified-SOTA recipe, in
// full" (manifest SLIDING_WINDOW, SPECULATIVE_CONFIG; "What each piece does, and
// why": decode is bound by the KV cache's bandwidth, which is what this measures).

#include <hip/hip_runtime.h>

#include "kv_access.h"
#include "swattn.h"
#include "swattn_internal.h"

namespace swattn {
namespace {

// 16 waves: a CU's load rate grows with the number of waves issuing loads (the verify
// step at four workgroups per unit: 6.0 us with 4 waves, 5.0 us with 16; the batched
// workloads, which fill HBM either way, are unchanged)
constexpr int kGatherThreads = 1024;
constexpr int kGatherLdsB = 64 * 1024;       // landing buffer (overwritten freely)
constexpr int kGatherMaxRows = 1024;         // window rows of one workgroup (offsets in LDS)
constexpr int kGatherMaxQRows = 512;         // Q rows of one workgroup

#define LDS_ADDR(p) ((__attribute__((address_space(3))) void*)(p))

// With the non-temporal cache policy, as the partition kernels' copies (64-row chunks
// aside), which measured faster on every launch that reads each row once.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void gather16(const void* src, const void* lds_dst) {
    const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)LDS_ADDR(lds_dst));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(a), "v"(src) : "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void gather_wait() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

struct GatherParams {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* block_table;
    const int32_t* ctx_len;
    void* out;
    int32_t Hkv, G, H, D, bs, max_blocks, num_blocks, max_ctx, n_q, window;
    int32_t kv_elt, q_elt, out_elt;
    int32_t lg_cpr, lg_qcpr;              // log2 of the 16-byte chunks of a cache row / a Q row
    int32_t parts;                        // workgroups per (problem, KV head)
};

__global__ __launch_bounds__(kGatherThreads) void window_gather_kernel(GatherParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char buf[kGatherLdsB];
    // byte offset of every row this workgroup reads: the window's K rows (V rows sit at
    // the same offsets in the V cache), then its Q rows
    __shared__ int64_t rowoff[kGatherMaxRows + kGatherMaxQRows];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int unit = blockIdx.x / p.parts, part = blockIdx.x % p.parts;
    const int b = unit / p.Hkv, g = unit % p.Hkv;
    const int ctx = p.ctx_len[b];
    const bool ok = ctx >= p.n_q && ctx <= p.max_blocks * p.bs && ctx <= p.max_ctx;
    const int u_hi = ok ? ctx : 0;                                    // one past the last key
    const int u_lo = ok ? max(0, ctx - p.n_q - p.window + 1) : 0;
    const int n_all = min(u_hi - u_lo, kGatherMaxRows);
    const int q_all = min(p.n_q * p.G, kGatherMaxQRows);
    // this workgroup's slices: window rows [w0, w0 + nrows), Q and output rows [r0, r0 + q_rows)
    const int w0 = n_all * part / p.parts, nrows = n_all * (part + 1) / p.parts - w0;
    const int r0 = q_all * part / p.parts, q_rows = q_all * (part + 1) / p.parts - r0;
    const int row_b = p.D * p.kv_elt;                                 // bytes per cache row
    for (int t = tid; t < nrows; t += kGatherThreads) {
        const int j = u_lo + w0 + t;
        const int blk = j / p.bs;
        const int phys = p.block_table[(int64_t)b * p.max_blocks + blk];
        // a row in an out-of-range block is read from row 0 instead (same byte count)
        rowoff[t] = phys >= 0 && phys < p.num_blocks ? ((int64_t)(phys * p.Hkv + g) * p.bs + (j - blk * p.bs)) * row_b
                                                     : 0;
    }
    for (int r = tid; r < q_rows; r += kGatherThreads) {
        const int i = (r0 + r) / p.G, h = g * p.G + (r0 + r - i * p.G);
        rowoff[kGatherMaxRows + r] = (((int64_t)b * p.n_q + i) * p.H + h) * (p.D * p.q_elt);
    }
    __syncthreads();

    // the unit's output rows: zeros, with 16-byte stores issued ahead of the loads
    const int o_cpr = p.D * p.out_elt / 16;
    unsigned char* obase = reinterpret_cast<unsigned char*>(p.out);
    for (int c = tid; c < q_rows * o_cpr; c += kGatherThreads) {
        const int r = c / o_cpr, col = c - r * o_cpr;
        *reinterpret_cast<uint4*>(obase + rowoff[kGatherMaxRows + r] / p.q_elt * p.out_elt + col * 16) =
            make_uint4(0u, 0u, 0u, 0u);
    }

    const int lg = p.lg_cpr;                                          // log2 of 16-byte chunks per row
    const int lgq = p.lg_qcpr;
    const int kv_chunks = nrows << lg;                                // per tensor
    const int total = 2 * kv_chunks + (q_rows << lgq);
    const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k);
    const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v);
    const unsigned char* qbase = reinterpret_cast<const unsigned char*>(p.q);
    int issued = 0;
    // chunk c = (i * waves + wave) * 64 + lane: lane l of a load writes LDS bytes 16 l of
    // a wave-uniform 1 KiB slot
    for (int base = wave * 64; base < total; base += kGatherThreads) {
        const int c = base + lane;
        const unsigned char* src = kbase;                             // a valid address for idle lanes
        if (c < 2 * kv_chunks) {
            const bool is_v = c >= kv_chunks;
            const int cc = is_v ? c - kv_chunks : c;
            src = (is_v ? vbase : kbase) + rowoff[cc >> lg] + ((cc & ((1 << lg) - 1)) << 4);
        } else if (c < total) {
            const int cc = c - 2 * kv_chunks;
            src = qbase + rowoff[kGatherMaxRows + (cc >> lgq)] + ((cc & ((1 << lgq) - 1)) << 4);
        }
        gather16(src, buf + (base % (kGatherLdsB / 16)) * 16);      // a 1 KiB slot inside buf
        if (++issued >= 48) {                                         // vmcnt holds at most 63
            gather_wait<32>();
            issued = 32;
        }
    }
    gather_wait<0>();
    __syncthreads();
}

// A plain contiguous read, the other reference point: the same number of bytes as a
// call moves, streamed by every CU from the first cycle (no table lookups before the
// first request, no per-unit workgroups).  Thread t of the grid reads 16-byte chunks
// t, t + T, t + 2T, ... (T threads in the grid), four in flight per round, with the
// non-temporal cache policy; each workgroup writes the xor of the chunks it read, so
// that a caller can check every byte was read, unless it is given no xor buffer (then
// nothing is written: the final store's latency is no part of a read floor).
constexpr int kReadThreads = 1024;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Xor over the wave's 64 lanes, wave-uniform: DPP moves within each 16-lane row (lane
// l ^ 1, l ^ 2, then rotations by 4 and 8), then the four rows' first lanes.  A shuffle
// per step would be an LDS round trip each (24 of them for four words), which at a few
// chunks per thread is longer than the reads.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_xor(uint32_t x) {
    x ^= dpp_u32<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    x ^= dpp_u32<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    x ^= dpp_u32<0x124>(x);   // row_ror:4
    x ^= dpp_u32<0x128>(x);   // row_ror:8
    return __builtin_amdgcn_readlane(x, 0) ^ __builtin_amdgcn_readlane(x, 16) ^ __builtin_amdgcn_readlane(x, 32) ^
           __builtin_amdgcn_readlane(x, 48);
}

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4_t* __restrict__ src, int64_t n16,
                                                                    uint32_t* __restrict__ xor_out) {
    __shared__ u32x4_t part[kReadThreads / 64];
    const int64_t stride = (int64_t)gridDim.x * kReadThreads;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
        const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= (a ^ b) ^ (c ^ d);
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
    if (xor_out == nullptr) return;   // the timing form: the reads alone (grid-uniform)
    u32x4_t wx;
#pragma unroll
    for (int e = 0; e < 4; ++e) wx[e] = wave_xor(acc[e]);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) part[wave] = wx;
    __syncthreads();
    if (threadIdx.x < 4) {
        uint32_t r = 0;
#pragma unroll
        for (int w = 0; w < kReadThreads / 64; ++w) r ^= part[w][threadIdx.x];
        xor_out[(int64_t)blockIdx.x * 4 + threadIdx.x] = r;
    }
}

}  // namespace
}  // namespace swattn

extern "C" swattn_status_t swattn_stream_read(const void* src, int64_t bytes, int32_t grid, uint32_t* xor_out,
                                              void* stream) {
    using namespace swattn;
    if (!src) return SWATTN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(xor_out) & 3) != 0)
        return SWATTN_ERR_ALIGN;
    if (bytes < 0 || bytes % 16 != 0 || grid < 1 || grid > 65536) return SWATTN_ERR_ARG;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kReadThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const u32x4_t*>(src), bytes / 16,
                       xor_out);
    return hipGetLastError() == hipSuccess ? SWATTN_OK : SWATTN_ERR_HIP;
}

extern "C" swattn_status_t swattn_window_gather(const swattn_desc_t* d, const void* q, const void* k_cache,
                                                const void* v_cache, const int32_t* block_table,
                                                const int32_t* ctx_len, int32_t n_q, int32_t window, int32_t parts,
                                                void* out, void* stream) {
    using namespace swattn;
    swattn_plan_t plan;
    swattn_status_t st = make_plan(d, n_q, window, SWATTN_MAX_NQ, &plan);   // the same argument checks
    if (st != SWATTN_OK) return st;
    if (!q || !k_cache || !v_cache || !block_table || !ctx_len || !out) return SWATTN_ERR_NULL;
    if (parts < 1 || parts > 16) return SWATTN_ERR_ARG;
    const auto al = [](const void* x, uintptr_t a) { return (reinterpret_cast<uintptr_t>(x) & (a - 1)) == 0; };
    if (!al(q, 16) || !al(k_cache, 16) || !al(v_cache, 16) || !al(out, 16) || !al(block_table, 4) || !al(ctx_len, 4))
        return SWATTN_ERR_ALIGN;
    GatherParams p;
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.block_table = block_table;
    p.ctx_len = ctx_len;
    p.out = out;
    p.Hkv = d->num_kv_heads;
    p.G = d->num_heads / d->num_kv_heads;
    p.H = d->num_heads;
    p.D = d->head_dim;
    p.bs = d->block_size;
    p.max_blocks = d->max_blocks_per_seq;
    p.num_blocks = d->num_blocks;
    p.max_ctx = d->max_ctx_len;
    p.n_q = n_q;
    p.window = window;
    p.kv_elt = d->kv_dtype == SWATTN_FP8_E4M3 ? 1 : (d->kv_dtype == SWATTN_BF16 ? 2 : 4);
    p.q_elt = d->q_dtype == SWATTN_F32 ? 4 : 2;
    p.out_elt = d->out_dtype == SWATTN_F32 ? 4 : 2;
    p.lg_cpr = 0;
    while ((16 << p.lg_cpr) < p.D * p.kv_elt) ++p.lg_cpr;      // rows are 64 * 2^k bytes
    p.lg_qcpr = 0;
    while ((16 << p.lg_qcpr) < p.D * p.q_elt) ++p.lg_qcpr;
    p.parts = parts;
    const int64_t grid = (int64_t)d->batch * d->num_kv_heads * parts;
    if (grid > INT32_MAX) return SWATTN_ERR_SHAPE;
    hipLaunchKernelGGL(window_gather_kernel, dim3((unsigned)grid), dim3(kGatherThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), p);
    return hipGetLastError() == hipSuccess ? SWATTN_OK : SWATTN_ERR_HIP;
}
