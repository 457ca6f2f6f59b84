// Split-KV partition kernel on gfx950 matrix cores (bf16 MFMA 16x16x32).
//
// One workgroup (4 waves) owns one (problem b, KV head g, 32-row chunk, KV
// split s).  A KV head's query rows are its n_q queries times the H/Hkv heads
// that share it (row r = i * G + head-in-group), so a verify step with n_q = 8
// and GQA 4 is one dense 32-row tile.  The split's keys are walked in tiles of
// 64 with an online softmax; within a tile:
//
//   phase A  wave w scores keys 16w..16w+15 of the tile for all 32 rows:
//            S^T = K . Q^T, K rows straight from HBM as the A operand, Q^T read
//            from the workgroup's Q rows in LDS.  The window mask (t - W, t] and the softmax scale are
//            applied and S goes to LDS; the wave also stages V of its 16 keys
//            into LDS transposed (V^T[d][key]), then issues the loads of its
//            next tile so they overlap the rest of this one.
//   phase B  each wave takes 8 rows (8 lanes per row): tile max, running max and
//            rescale factor, P = 2^(S - max) split into two bf16 terms (hi + lo)
//            written over S, running sum.
//   phase C  wave w owns D/4 output columns: O^T = alpha * O^T + V^T . P^T.
//
// Every wave loads only its own keys; Q is read from HBM once per workgroup.
// The workgroup writes the final output (S == 1) or a normalised partial and its
// log2-sum-exp for the merge kernel (S > 1).
//
// Semantics follow "The Fast Gemma Challenge: our verified-SOTA recipe, in full"
// (manifest: SLIDING_WINDOW, SPECULATIVE_CONFIG, SPLITKV_VERIFY,
// SPLITKV_VERIFY_MAX_Q; "What each piece does, and why"): each query attends to
// the most recent W positions up to its own, the target and drafts of one step
// are scored together, and a long KV range is split across workgroups.

#include <hip/hip_runtime.h>

#include "kv_access.h"
#include "swattn_internal.h"

namespace swattn {
namespace {

constexpr int kT = kMfmaTileKeys;           // 64 keys per tile
constexpr int kVtStride = kT + 8;           // bf16 per V^T row (144 B, 16-byte aligned rows)
constexpr int kSStride = kT + 4;            // floats per S row (272 B); P hi/lo overwrite it in place

template <int D>
struct MfmaLds {
    static constexpr int kVtBytes = D * kVtStride * 2;
    static constexpr int kQStride = D + 8;  // bf16 per staged Q row
    static constexpr int kQBytes = kMfmaRows * kQStride * 2;
    static constexpr int kSBytes = kMfmaRows * kSStride * 4;
    static constexpr int kRowIdxBytes = kMfmaMaxKeys * 4;
    static constexpr int kMiscBytes = 3 * kMfmaRows * 4;   // alpha, final max, final sum
    static constexpr int kTableBytes = kMfmaThreads * 4;   // block-table row (short rows only)
    static constexpr int kBytes = kVtBytes + kQBytes + kSBytes + kRowIdxBytes + kMiscBytes + kTableBytes;
};

__device__ __forceinline__ f32x4_t mfma_bf16(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Lane moves inside groups of 8 lanes (gfx9 data-parallel-primitive encodings).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- lane 7-i within 8

__device__ __forceinline__ float max8(float x) {     // every lane of an aligned group of 8 gets the max
    x = fmaxf(x, dpp<kDppXor1>(x));
    x = fmaxf(x, dpp<kDppXor2>(x));
    return fmaxf(x, dpp<kDppHalfMirror>(x));
}

__device__ __forceinline__ float sum8(float x) {
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    return x + dpp<kDppHalfMirror>(x);
}

// Key-group swizzle of the V^T rows: groups of 4 keys are XOR-ed with an even
// value below 16 taken from the row's 8-dim chunk.  It spreads the transposing
// writes over the LDS banks and keeps each aligned pair of groups contiguous.
__device__ __forceinline__ int vt_group(int group, int d) { return group ^ (((d >> 3) & 7) << 1); }

template <int D, bool FP8, bool OUT_F32>
__global__ __launch_bounds__(kMfmaThreads) void partition_mfma_kernel(PartitionParams p) {
    using L = MfmaLds<D>;
    constexpr int KS = D / 32;                   // 32-dim k-steps of S^T = K Q^T
    constexpr int DC = D / 8;                    // 8-element chunks per row
    constexpr int VITEMS = 4 * DC;               // (key quad, chunk) pairs of a wave's 16 keys
    constexpr int VIT = (VITEMS + kWaveSize - 1) / kWaveSize;
    constexpr int DTW = D / 64;                  // 16-column tiles per wave in phase C

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::kBytes];
    uint16_t* vt = reinterpret_cast<uint16_t*>(smem);
    uint16_t* qs = reinterpret_cast<uint16_t*>(smem + L::kVtBytes);    // Q rows, read as Q^T operands
    float* sbuf = reinterpret_cast<float*>(smem + L::kVtBytes + L::kQBytes);
    int* rowidx = reinterpret_cast<int*>(smem + L::kVtBytes + L::kQBytes + L::kSBytes);
    float* alpha_s = reinterpret_cast<float*>(rowidx + kMfmaMaxKeys);
    float* st_m = alpha_s + kMfmaRows;
    float* st_l = st_m + kMfmaRows;
    int* tbl = reinterpret_cast<int*>(st_l + kMfmaRows);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int q4 = lane >> 4;

    int lin = blockIdx.x;
    const int s = lin % p.S;
    lin /= p.S;
    const int rc = lin % p.row_chunks;
    lin /= p.row_chunks;
    const int g = lin % p.Hkv;
    const int b = lin / p.Hkv;

    // A block-table row that fits one entry per thread is read while ctx_len is in
    // flight, which removes one dependent round trip to memory.
    const bool short_row = p.max_blocks <= kMfmaThreads;
    const int tb = (short_row && tid < p.max_blocks) ? p.block_table[(int64_t)b * p.max_blocks + tid] : 0;
    const int ctx = p.ctx_len[b];
    const bool seq_ok = ctx >= p.n_q && ctx <= p.max_blocks * p.bs && ctx <= p.max_ctx;
    const int pos0 = seq_ok ? ctx - p.n_q : 0;             // position of query 0
    const int u_lo = max(0, pos0 - p.window + 1);          // first key of the step's union window
    int k0 = 0, nk = 0;
    if (seq_ok) {
        const int kps = (ctx - u_lo + p.S - 1) / p.S;
        k0 = u_lo + s * kps;
        nk = max(0, min(ctx, k0 + kps) - k0);              // <= kMfmaMaxKeys by the plan
    }
    const int ntiles = (nk + kT - 1) / kT;

    if (short_row) {
        tbl[tid] = tb;
        __syncthreads();
    }

    // ---- key -> cache row (phys * Hkv + g) * bs + off; -1 bad block id, -2 no key -----
    for (int t = tid; t < kMfmaMaxKeys; t += kMfmaThreads) {
        int ri = -2;
        if (t < nk) {
            const int j = k0 + t;
            const int blk = p.bs_log2 >= 0 ? j >> p.bs_log2 : j / p.bs;
            const int off = j - blk * p.bs;
            const int phys = short_row ? tbl[blk] : p.block_table[(int64_t)b * p.max_blocks + blk];
            ri = (phys >= 0 && phys < p.num_blocks) ? (phys * p.Hkv + g) * p.bs + off : -1;
        }
        rowidx[t] = ri;
    }

    // ---- Q rows of this chunk -> LDS (coalesced 16-byte loads, zero past R) ---------
    const uint16_t* qg = reinterpret_cast<const uint16_t*>(p.q);
    for (int item = tid; item < kMfmaRows * DC; item += kMfmaThreads) {
        const int row = item / DC, c = item - row * DC;
        const int r = rc * kMfmaRows + row;
        const bool rv = r < p.R;
        const int i = rv ? r / p.G : 0;
        const int h = g * p.G + (rv ? r - i * p.G : 0);
        const uint4 v = ld_global_16(qg + (((int64_t)b * p.n_q + i) * p.H + h) * D + c * 8);
        *reinterpret_cast<uint4*>(qs + row * L::kQStride + c * 8) = rv ? v : make_uint4(0, 0, 0, 0);
    }

    // each lane's two query rows (phase A / C layout) and their windows
    int row_lo[2], row_hi[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = rc * kMfmaRows + rt * 16 + l16;
        const bool rv = r < p.R;
        const int i = rv ? r / p.G : 0;
        row_lo[rt] = rv ? max(0, pos0 + i - p.window + 1) : 1;
        row_hi[rt] = rv ? pos0 + i : 0;
    }
    float scale_log2 = p.scale_log2;
    float out_scale = 1.0f;
    if constexpr (FP8) {
        scale_log2 *= p.k_scale[g];
        out_scale = p.v_scale[g];
    }
    __syncthreads();
    const uint16_t* qop = qs + l16 * L::kQStride + q4 * 8;   // this lane's Q^T operand row

    const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k);
    const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v);
    const uint4 zero8 = make_uint4(0, 0, 0, 0);
    const uint4 nan8 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);

    // ---- per-wave tile loads: K as the A operand, V chunks for the transpose --------
    uint4 kreg[KS];
    uint4 vreg[VIT][4];
    int vri[VIT][4];
    auto load_tile = [&](int t) {
        const int kri = rowidx[t * kT + wave * 16 + l16];
        const int64_t ke = (int64_t)max(kri, 0) * D + q4 * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (FP8)
                kreg[ks] = e4m3x8_to_bf16x8(ld_global_8(kbase + ke + ks * 32));
            else
                kreg[ks] = ld_global_16(kbase + (ke + ks * 32) * 2);
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int item = lane + kWaveSize * it;
            const bool item_ok = item < VITEMS;
            const int kqd = item & 3, dc = item_ok ? item >> 2 : 0;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int ri = item_ok ? rowidx[t * kT + wave * 16 + kqd * 4 + kk] : -2;
                vri[it][kk] = ri;
                const int64_t ve = (int64_t)max(ri, 0) * D + dc * 8;
                if constexpr (FP8)
                    vreg[it][kk] = e4m3x8_to_bf16x8(ld_global_8(vbase + ve));
                else
                    vreg[it][kk] = ld_global_16(vbase + ve * 2);
            }
        }
    };

    float m_run = -INFINITY, l_run = 0.0f;   // phase-B lanes: row wave*8 + lane/8
    f32x4_t o[DTW][2];
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt) o[dt][0] = o[dt][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int brow = wave * 8 + (lane >> 3);
    const int bcol = (lane & 7) * 8;
    const int dbase = wave * DTW * 16;

    if (ntiles > 0) load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
        // ---- phase A: scores of this wave's 16 keys; V^T staging; next tile's loads
        // Keys without a cache row were loaded from row 0: their scores are masked
        // below (a select, so whatever row 0 holds cannot leak); a bad block id
        // turns the key's score into NaN.
        const int4 kr4 = *reinterpret_cast<const int4*>(rowidx + t * kT + wave * 16 + q4 * 4);
        const int krs[4] = {kr4.x, kr4.y, kr4.z, kr4.w};
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc = mfma_bf16(kreg[ks], *reinterpret_cast<const uint4*>(qop + rt * 16 * L::kQStride + ks * 32), acc);
            // lane holds S^T[key t*64 + wave*16 + q4*4 + e][row rt*16 + l16]
            float4 sv;
            float* svp = reinterpret_cast<float*>(&sv);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tt = t * kT + wave * 16 + q4 * 4 + e;
                const int j = k0 + tt;
                const bool ok = tt < nk && j >= row_lo[rt] && j <= row_hi[rt];
                const float sc = krs[e] == -1 ? __builtin_nanf("") : acc[e] * scale_log2;
                svp[e] = ok ? sc : -INFINITY;
            }
            *reinterpret_cast<float4*>(sbuf + (rt * 16 + l16) * kSStride + wave * 16 + q4 * 4) = sv;
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int item = lane + kWaveSize * it;
            if (item >= VITEMS) continue;
            const int kqd = item & 3, dc = item >> 2;
            uint4 w4[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                w4[kk] = vri[it][kk] >= 0 ? vreg[it][kk] : (vri[it][kk] == -1 ? nan8 : zero8);
            const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&w4[0]);
            const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&w4[1]);
            const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&w4[2]);
            const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&w4[3]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int wi = e >> 1;
                uint2 pk;
                if (e & 1) {
                    pk.x = (w0[wi] >> 16) | (w1[wi] & 0xFFFF0000u);
                    pk.y = (w2[wi] >> 16) | (w3[wi] & 0xFFFF0000u);
                } else {
                    pk.x = (w0[wi] & 0xFFFFu) | (w1[wi] << 16);
                    pk.y = (w2[wi] & 0xFFFFu) | (w3[wi] << 16);
                }
                const int d = dc * 8 + e;
                *reinterpret_cast<uint2*>(vt + d * kVtStride + vt_group(wave * 4 + kqd, d) * 4) = pk;
            }
        }
        if (t + 1 < ntiles) load_tile(t + 1);
        __syncthreads();

        // ---- phase B: running max / sum of 8 rows per wave, P (hi, lo) over S --------
        {
            float* srow = sbuf + brow * kSStride;
            const float4 a0 = *reinterpret_cast<const float4*>(srow + bcol);
            const float4 a1 = *reinterpret_cast<const float4*>(srow + bcol + 4);
            const float sv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            float mt = sv[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sv[e]);
            mt = max8(mt);
            const float m_new = fmaxf(m_run, mt);
            const float mu = m_new == -INFINITY ? 0.0f : m_new;
            const float alpha = exp2f(m_run - mu);
            float psum = 0.0f;
            uint32_t ph[4], pl[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const float p0 = exp2f(sv[2 * e2] - mu);
                const float p1 = exp2f(sv[2 * e2 + 1] - mu);
                const uint32_t h0 = f32_to_bf16_bits(p0), h1 = f32_to_bf16_bits(p1);
                const uint32_t r0 = f32_to_bf16_bits(p0 - bf16_bits_to_f32(h0));
                const uint32_t r1 = f32_to_bf16_bits(p1 - bf16_bits_to_f32(h1));
                psum += p0 + p1;
                ph[e2] = h0 | (h1 << 16);
                pl[e2] = r0 | (r1 << 16);
            }
            l_run = l_run * alpha + sum8(psum);
            m_run = m_new;
            uint16_t* prow = reinterpret_cast<uint16_t*>(srow);
            *reinterpret_cast<uint4*>(prow + bcol) = make_uint4(ph[0], ph[1], ph[2], ph[3]);
            *reinterpret_cast<uint4*>(prow + kT + bcol) = make_uint4(pl[0], pl[1], pl[2], pl[3]);
            if ((lane & 7) == 0) alpha_s[brow] = alpha;
        }
        __syncthreads();

        // ---- phase C: O^T = alpha O^T + V^T P^T over this tile -----------------------
        {
            const float a0 = alpha_s[l16], a1 = alpha_s[16 + l16];
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt) {
                o[dt][0] *= a0;
                o[dt][1] *= a1;
            }
#pragma unroll
            for (int ks2 = 0; ks2 < kT / 32; ++ks2) {
                uint4 bh[2], bl[2];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const uint16_t* prow = reinterpret_cast<const uint16_t*>(sbuf + (rt * 16 + l16) * kSStride);
                    bh[rt] = *reinterpret_cast<const uint4*>(prow + ks2 * 32 + q4 * 8);
                    bl[rt] = *reinterpret_cast<const uint4*>(prow + kT + ks2 * 32 + q4 * 8);
                }
#pragma unroll
                for (int dt = 0; dt < DTW; ++dt) {
                    const int d = dbase + dt * 16 + l16;
                    const uint4 a = *reinterpret_cast<const uint4*>(vt + d * kVtStride +
                                                                   vt_group(ks2 * 8 + q4 * 2, d) * 4);
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) {
                        o[dt][rt] = mfma_bf16(a, bh[rt], o[dt][rt]);
                        o[dt][rt] = mfma_bf16(a, bl[rt], o[dt][rt]);
                    }
                }
            }
        }
        if (t + 1 < ntiles) __syncthreads();   // S and V^T are rewritten by the next tile
    }

    if ((lane & 7) == 0) {
        st_m[brow] = m_run;
        st_l[brow] = l_run;
    }
    __syncthreads();

    // ---- epilogue: lane holds O^T[d = dbase + dt*16 + q4*4 + e][row rt*16 + l16] -----
    const float poison = seq_ok ? 0.0f : __builtin_nanf("");
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int row = rt * 16 + l16;
        const int r = rc * kMfmaRows + row;
        if (r >= p.R) continue;
        const float Lr = st_l[row];
        const float inv = Lr == 0.0f ? 0.0f : out_scale / Lr;   // a NaN sum must propagate
        if (p.S == 1) {
            const int i = r / p.G;
            const int h = g * p.G + (r - i * p.G);
            const int64_t base = (((int64_t)b * p.n_q + i) * p.H + h) * D + dbase + q4 * 4;
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt) {
                const f32x4_t v = o[dt][rt] * inv + poison;
                if constexpr (OUT_F32) {
                    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.out) + base + dt * 16) = v;
                } else {
                    uint2 w;
                    w.x = pack_bf16x2(v[0], v[1]);
                    w.y = pack_bf16x2(v[2], v[3]);
                    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + base + dt * 16) = w;
                }
            }
        } else {
            const int64_t prow = (((int64_t)b * p.Hkv + g) * p.S + s) * p.R + r;
            float* dst = p.ws_o + prow * D + dbase + q4 * 4;
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt)
                *reinterpret_cast<f32x4_t*>(dst + dt * 16) = o[dt][rt] * inv + poison;
            if (wave == 0 && q4 == 0)
                p.ws_lse[prow] = (Lr == 0.0f ? -INFINITY : st_m[row] + log2f(Lr)) + poison;
        }
    }
}

template <int D>
int launch_d(const PartitionParams& p, int grid, hipStream_t st) {
    const bool fp8 = p.kv_dtype == SWATTN_FP8_E4M3;
    const bool of32 = p.out_dtype == SWATTN_F32;
    const dim3 blk(kMfmaThreads);
    if (fp8 && of32)
        hipLaunchKernelGGL((partition_mfma_kernel<D, true, true>), dim3(grid), blk, 0, st, p);
    else if (fp8)
        hipLaunchKernelGGL((partition_mfma_kernel<D, true, false>), dim3(grid), blk, 0, st, p);
    else if (of32)
        hipLaunchKernelGGL((partition_mfma_kernel<D, false, true>), dim3(grid), blk, 0, st, p);
    else
        hipLaunchKernelGGL((partition_mfma_kernel<D, false, false>), dim3(grid), blk, 0, st, p);
    return (int)hipGetLastError();
}

}  // namespace

int launch_partition_mfma(const PartitionParams& p, int grid, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    switch (p.D) {
        case 64: return launch_d<64>(p, grid, st);
        case 128: return launch_d<128>(p, grid, st);
        case 256: return launch_d<256>(p, grid, st);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace swattn
