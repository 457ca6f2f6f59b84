// Split-KV partition kernel on gfx950 matrix cores (bf16 MFMA 16x16x32).
//
// One workgroup (4 waves) owns one (problem b, KV head g, row chunk, KV split s).
// The query rows of a KV head are the n_q queries times the H/Hkv heads that
// share it (row r = i * G + head-in-group), so a verify step with n_q = 8 and
// GQA 4 gives a dense 32-row tile.  Each wave owns 32 rows (two 16-row tiles)
// and a strided subset of the split's 32-key chunks:
//
//   S^T (keys x rows) = K . Q^T      A = K rows straight from HBM (16 B per lane),
//                                    B = Q^T held in registers for the whole call
//   mask to -inf outside each query's window (t - W, t], online softmax in the
//   exp2 domain, P split into two bf16 terms (hi + lo)
//   O^T (dims x rows) += V^T . P^T   A = V^T from a per-wave LDS transpose,
//                                    B = P^T straight from the S^T accumulators
//
// Working in the transposed orientation puts one query row per lane column, so
// the row max/sum need two cross-lane steps and the rescale of O needs none.
// Waves that split a row chunk's keys are merged through LDS at the end; the
// workgroup then writes the final output (S == 1) or a normalised partial and
// its log2-sum-exp for the merge kernel (S > 1).
//
// Semantics follow "The Fast Gemma Challenge: our verified-SOTA recipe, in full"
// (manifest: SLIDING_WINDOW, SPECULATIVE_CONFIG, SPLITKV_VERIFY,
// SPLITKV_VERIFY_MAX_Q; "What each piece does, and why"): each query attends to
// the most recent W positions up to its own, the target and drafts of one step
// are scored together, and the KV range is split across workgroups.

#include <hip/hip_runtime.h>

#include "kv_access.h"
#include "swattn_internal.h"

namespace swattn {
namespace {

constexpr int kVtPad = 4;                                   // bf16 elements of padding per V^T row
constexpr int kVtStride = kMfmaChunkKeys + kVtPad;          // 36 elements = 72 B
constexpr int kMergeCols = 64;                              // d columns merged per LDS pass
constexpr int kMergeStride = kMergeCols + 4;                // floats per merge-buffer row

template <int D>
struct MfmaLds {
    static constexpr int kVtBytes = 4 * D * kVtStride * 2;
    static constexpr int kMergeBytes = 3 * kMfmaRowsPerWave * kMergeStride * 4;
    static constexpr int kBytes = kVtBytes > kMergeBytes ? kVtBytes : kMergeBytes;
};

__device__ __forceinline__ f32x4_t mfma_bf16(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max_q(float x) {   // reduce over lanes l, l^16, l^32, l^48
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

__device__ __forceinline__ float wave_sum_q(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// Element offset of position j of KV head g, or -1 when its block id is out of range.
__device__ __forceinline__ int64_t kv_row_offset(const PartitionParams& p, int b, int g, int j) {
    const int blk = j / p.bs;
    const int off = j - blk * p.bs;
    const int phys = p.block_table[(int64_t)b * p.max_blocks + blk];
    if (phys < 0 || phys >= p.num_blocks) return -1;
    return (((int64_t)phys * p.Hkv + g) * p.bs + off) * (int64_t)p.D;
}

template <int D, bool FP8, bool OUT_F32>
__global__ __launch_bounds__(kBlockThreads) void partition_mfma_kernel(PartitionParams p) {
    constexpr int KS = D / 32;        // 32-dim k-steps of S^T = K Q^T
    constexpr int DT = D / 16;        // 16-dim tiles of O^T
    constexpr int DC = D / 8;         // 8-element chunks of a row
    constexpr int VPASS = DC / 8;     // V staging passes (8 d-chunks x 8 key-quads per pass)
    constexpr int ELT = FP8 ? 1 : 2;  // bytes per cached K/V element

    __shared__ __attribute__((aligned(16))) unsigned char smem[MfmaLds<D>::kBytes];
    __shared__ float st_m[4][kMfmaRowsPerWave];
    __shared__ float st_l[4][kMfmaRowsPerWave];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l16 = lane & 15;
    const int q4 = lane >> 4;

    int lin = blockIdx.x;
    const int s = lin % p.S;
    lin /= p.S;
    const int rc = lin % p.row_chunks;
    lin /= p.row_chunks;
    const int g = lin % p.Hkv;
    const int b = lin / p.Hkv;

    const int RG = p.rows_per_chunk / kMfmaRowsPerWave;   // 1, 2 or 4 row groups
    const int KG = 4 / RG;                                // waves sharing a row group
    const int rg = wave % RG;
    const int kg = wave / RG;

    const int ctx = p.ctx_len[b];
    const bool seq_ok = ctx >= p.n_q && ctx <= p.max_blocks * p.bs && ctx <= p.max_ctx;
    const int pos0 = seq_ok ? ctx - p.n_q : 0;            // position of query 0
    const int u_lo = max(0, pos0 - p.window + 1);         // union of the step's windows
    const int u_hi = seq_ok ? ctx - 1 : -1;
    int cb = 0, ce = 0;
    if (seq_ok) {
        const int c_lo = u_lo / kMfmaChunkKeys;
        const int nch = u_hi / kMfmaChunkKeys - c_lo + 1;
        const int cps = (nch + p.S - 1) / p.S;
        cb = c_lo + s * cps;
        ce = min(c_lo + nch, cb + cps);
    }

    // ---- this lane's query rows and their windows -------------------------------
    const int row_base = rc * p.rows_per_chunk + rg * kMfmaRowsPerWave;
    int row_lo[2], row_hi[2];
    uint4 qreg[2][KS];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = row_base + rt * 16 + l16;
        const bool rv = r < p.R;
        const int i = rv ? r / p.G : 0;
        const int h = g * p.G + (rv ? r - i * p.G : 0);
        row_lo[rt] = rv ? max(0, pos0 + i - p.window + 1) : 1;
        row_hi[rt] = rv ? pos0 + i : 0;
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) +
                             (((int64_t)b * p.n_q + i) * p.H + h) * D + q4 * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qreg[rt][ks] = rv ? ld_global_16(qp + ks * 32) : make_uint4(0, 0, 0, 0);
    }

    float scale_log2 = p.scale_log2;
    float out_scale = 1.0f;
    if constexpr (FP8) {
        scale_log2 *= p.k_scale[g] * 256.0f;
        out_scale = p.v_scale[g] * 256.0f;
    }

    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.0f, 0.0f};
    f32x4_t o[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        o[dt][0] = o[dt][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    uint16_t* vt = reinterpret_cast<uint16_t*>(smem) + wave * D * kVtStride;
    const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k);
    const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v);
    const uint4 nan8 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
    const uint4 zero8 = make_uint4(0, 0, 0, 0);

    for (int c = cb + kg; c < ce; c += KG) {
        const int key0 = c * kMfmaChunkKeys;

        // ---- K tile: A operand of S^T, lane holds key (kt*16 + l16), dims q4*8.. of each k-step
        uint4 kreg[2][KS];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int j = key0 + kt * 16 + l16;
            const bool in_union = j >= u_lo && j <= u_hi;
            const int64_t off = in_union ? kv_row_offset(p, b, g, j) : -1;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (!in_union) {
                    kreg[kt][ks] = zero8;
                } else if (off < 0) {
                    kreg[kt][ks] = nan8;
                } else if constexpr (FP8) {
                    kreg[kt][ks] = e4m3x8_to_bf16x8_div256(
                        ld_global_8(kbase + (off + ks * 32 + q4 * 8) * ELT));
                } else {
                    kreg[kt][ks] = ld_global_16(kbase + (off + ks * 32 + q4 * 8) * ELT);
                }
            }
        }

        // ---- V tile: HBM -> registers -> per-wave LDS as V^T[d][key]
        {
            const int kq = lane & 7;          // key quad: keys kq*4 .. kq*4+3
            const int dcl = lane >> 3;        // d-chunk within a pass
            int64_t voff[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int j = key0 + kq * 4 + kk;
                voff[kk] = (j >= u_lo && j <= u_hi) ? kv_row_offset(p, b, g, j) : -2;
            }
#pragma unroll
            for (int ps = 0; ps < VPASS; ++ps) {
                const int dc = ps * 8 + dcl;
                uint4 vr[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    if (voff[kk] == -2) {
                        vr[kk] = zero8;
                    } else if (voff[kk] < 0) {
                        vr[kk] = nan8;
                    } else if constexpr (FP8) {
                        vr[kk] = e4m3x8_to_bf16x8_div256(ld_global_8(vbase + (voff[kk] + dc * 8) * ELT));
                    } else {
                        vr[kk] = ld_global_16(vbase + (voff[kk] + dc * 8) * ELT);
                    }
                }
                const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vr[0]);
                const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vr[1]);
                const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vr[2]);
                const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vr[3]);
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
                    *reinterpret_cast<uint2*>(vt + (dc * 8 + e) * kVtStride + kq * 4) = pk;
                }
            }
        }

        // ---- S^T = K Q^T : lane holds keys kt*16 + q4*4 + e for row tile rt, row l16
        f32x4_t sacc[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = mfma_bf16(kreg[kt][ks], qreg[rt][ks], acc);
                sacc[kt][rt] = acc;
            }

        // ---- window mask + online softmax (log2 domain); P^T as the B operand of PV
        uint4 pb[2], pb_lo[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float sv[2][4];
            float mloc = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = key0 + kt * 16 + q4 * 4 + e;
                    const bool ok = j >= row_lo[rt] && j <= row_hi[rt];
                    sv[kt][e] = ok ? sacc[kt][rt][e] * scale_log2 : -INFINITY;
                    mloc = fmaxf(mloc, sv[kt][e]);
                }
            mloc = wave_max_q(mloc);
            const float m_new = fmaxf(m_run[rt], mloc);
            const float m_use = m_new == -INFINITY ? 0.0f : m_new;
            const float alpha = exp2f(m_run[rt] - m_use);
            m_run[rt] = m_new;
            // P = hi + lo with hi, lo bf16: two PV products keep ~16 significant bits of
            // every weight, so the rounding of P stays far below the output tolerance.
            float psum = 0.0f;
            uint32_t ph[4], pl[4];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int e2 = 0; e2 < 2; ++e2) {
                    const float p0 = exp2f(sv[kt][2 * e2] - m_use);
                    const float p1 = exp2f(sv[kt][2 * e2 + 1] - m_use);
                    const uint32_t h0 = f32_to_bf16_bits(p0), h1 = f32_to_bf16_bits(p1);
                    const uint32_t r0 = f32_to_bf16_bits(p0 - bf16_bits_to_f32(h0));
                    const uint32_t r1 = f32_to_bf16_bits(p1 - bf16_bits_to_f32(h1));
                    psum += p0 + p1;
                    ph[kt * 2 + e2] = h0 | (h1 << 16);
                    pl[kt * 2 + e2] = r0 | (r1 << 16);
                }
            l_run[rt] = l_run[rt] * alpha + psum;
            pb[rt] = make_uint4(ph[0], ph[1], ph[2], ph[3]);
            pb_lo[rt] = make_uint4(pl[0], pl[1], pl[2], pl[3]);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= alpha;
        }

        // ---- O^T += V^T P^T : A lane holds V^T[d = dt*16 + l16][keys q4*4.. and 16 + q4*4..]
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const uint16_t* src = vt + (dt * 16 + l16) * kVtStride + q4 * 4;
            const uint2 a0 = *reinterpret_cast<const uint2*>(src);
            const uint2 a1 = *reinterpret_cast<const uint2*>(src + 16);
            const uint4 a = make_uint4(a0.x, a0.y, a1.x, a1.y);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                o[dt][rt] = mfma_bf16(a, pb[rt], o[dt][rt]);
                o[dt][rt] = mfma_bf16(a, pb_lo[rt], o[dt][rt]);
            }
        }
    }

    // ---- combine the waves that split this row group's keys ---------------------
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) l_run[rt] = wave_sum_q(l_run[rt]);

    float m_fin[2], l_fin[2];
    if (KG == 1) {
        m_fin[0] = m_run[0]; m_fin[1] = m_run[1];
        l_fin[0] = l_run[0]; l_fin[1] = l_run[1];
    } else {
        if (q4 == 0) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                st_m[wave][rt * 16 + l16] = m_run[rt];
                st_l[wave][rt * 16 + l16] = l_run[rt];
            }
        }
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float M = -INFINITY;
            for (int k = 0; k < KG; ++k) M = fmaxf(M, st_m[rg + k * RG][rt * 16 + l16]);
            const float Mu = M == -INFINITY ? 0.0f : M;
            float L = 0.0f;
            for (int k = 0; k < KG; ++k) {
                const int w = rg + k * RG;
                L += st_l[w][rt * 16 + l16] * exp2f(st_m[w][rt * 16 + l16] - Mu);
            }
            const float mine = exp2f(m_run[rt] - Mu);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= mine;
            m_fin[rt] = M;
            l_fin[rt] = L;
        }
        float* mbuf = reinterpret_cast<float*>(smem);
#pragma unroll
        for (int c0 = 0; c0 < D; c0 += kMergeCols) {
            __syncthreads();   // V^T reads / previous pass done before the buffer is overwritten
            if (kg > 0) {
                float* dst = mbuf + ((kg - 1) * RG + rg) * kMfmaRowsPerWave * kMergeStride;
#pragma unroll
                for (int dt = c0 / 16; dt < (c0 + kMergeCols) / 16; ++dt)
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
                        *reinterpret_cast<f32x4_t*>(dst + (rt * 16 + l16) * kMergeStride +
                                                    (dt * 16 - c0) + q4 * 4) = o[dt][rt];
            }
            __syncthreads();
            if (kg == 0) {
                for (int k = 1; k < KG; ++k) {
                    const float* src = mbuf + ((k - 1) * RG + rg) * kMfmaRowsPerWave * kMergeStride;
#pragma unroll
                    for (int dt = c0 / 16; dt < (c0 + kMergeCols) / 16; ++dt)
#pragma unroll
                        for (int rt = 0; rt < 2; ++rt)
                            o[dt][rt] += *reinterpret_cast<const f32x4_t*>(
                                src + (rt * 16 + l16) * kMergeStride + (dt * 16 - c0) + q4 * 4);
                }
            }
        }
    }
    if (kg != 0) return;

    // ---- epilogue: final output (S == 1) or normalised partial + log2-sum-exp --------
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = row_base + rt * 16 + l16;
        if (r >= p.R) continue;
        // l == 0: no key of this split is in the row's window; a NaN l must propagate.
        const float inv = l_fin[rt] == 0.0f ? 0.0f : out_scale / l_fin[rt];
        const float poison = seq_ok ? 0.0f : __builtin_nanf("");
        if (p.S == 1) {
            const int i = r / p.G;
            const int h = g * p.G + (r - i * p.G);
            const int64_t base = (((int64_t)b * p.n_q + i) * p.H + h) * D + q4 * 4;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
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
            float* dst = p.ws_o + prow * D + q4 * 4;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *reinterpret_cast<f32x4_t*>(dst + dt * 16) = o[dt][rt] * inv + poison;
            if (q4 == 0)
                p.ws_lse[prow] = (l_fin[rt] == 0.0f ? -INFINITY : m_fin[rt] + log2f(l_fin[rt])) + poison;
        }
    }
}

template <int D>
int launch_d(const PartitionParams& p, int grid, hipStream_t st) {
    const bool fp8 = p.kv_dtype == SWATTN_FP8_E4M3;
    const bool of32 = p.out_dtype == SWATTN_F32;
    if (fp8 && of32)
        hipLaunchKernelGGL((partition_mfma_kernel<D, true, true>), dim3(grid), dim3(kBlockThreads), 0, st, p);
    else if (fp8)
        hipLaunchKernelGGL((partition_mfma_kernel<D, true, false>), dim3(grid), dim3(kBlockThreads), 0, st, p);
    else if (of32)
        hipLaunchKernelGGL((partition_mfma_kernel<D, false, true>), dim3(grid), dim3(kBlockThreads), 0, st, p);
    else
        hipLaunchKernelGGL((partition_mfma_kernel<D, false, false>), dim3(grid), dim3(kBlockThreads), 0, st, p);
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
