// Split-KV partition kernel on gfx950 matrix cores (bf16 MFMA 16x16x32).
//
// One workgroup (4 waves) owns one (problem b, KV head g, 32-row chunk, KV
// split s).  A KV head's query rows are its n_q queries times the H/Hkv heads
// that share it (row r = i * G + head-in-group), so a verify step with n_q = 8
// and GQA 4 is one dense 32-row tile.  The split's keys are walked in tiles of
// 64 with an online softmax.  Per tile t:
//
//   phase A  wave w scores keys 16w..16w+15 for all 32 rows: S^T = K . Q^T with
//            the K rows as the A operand (registers, loaded one tile ahead) and
//            Q^T held in registers for the whole call.  The window mask
//            (t - W, t] and the softmax scale are applied; S goes to LDS.
//   phase B  the V rows of tile t+1 start streaming into LDS with direct
//            global-to-LDS loads (no registers, no VALU), then the K rows of tile
//            t+1 into registers; 8 lanes per row compute the running max, rescale
//            factor and P = 2^(S - max) as two bf16 terms (hi + lo) over S, and the
//            running sum.
//   phase C  wave w owns D/4 output columns: O^T = alpha O^T + V^T . P^T, with
//            V^T read from the row-major V tile by LDS transpose reads.
//
// V rows are stored with their 16-byte chunks XOR-swizzled by row so that the
// transpose reads of consecutive keys hit distinct LDS banks; absent keys and
// keys in a bad block read a zero row (a bad block's score is NaN).  The workgroup
// writes the final output (S == 1) or a normalised partial and its log2-sum-exp
// for the merge kernel (S > 1).
//
// Semantics follow "The Fast Gemma Challenge: our verified-SOTA recipe, in full"
// (manifest: SLIDING_WINDOW, SPECULATIVE_CONFIG, SPLITKV_VERIFY,
// SPLITKV_VERIFY_MAX_Q; "What each piece does, and why"): each query attends to
// the most recent W positions up to its own, the target and drafts of one step
// are scored together, and a long KV range is split across workgroups.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "kv_access.h"
#include "swattn_internal.h"

namespace swattn {
namespace {

constexpr int kT = kMfmaTileKeys;           // 64 keys per tile
constexpr int kSStride = kT + 4;            // floats per S row (272 B); P hi/lo overwrite it in place

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef int int2_t __attribute__((ext_vector_type(2)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

template <int D, bool FP8>
struct Geo {
    static constexpr int kElt = FP8 ? 1 : 2;
    static constexpr int kRowB = D * kElt;             // bytes per cache row
    static constexpr int kCpr = kRowB / 16;            // 16-byte chunks per row
    static constexpr int kRpi = 64 / kCpr;             // rows per 64-lane DMA instruction
    static constexpr int kNv = 16 / kRpi;              // DMA instructions per wave per tile
    static constexpr int kStage = kT * kRowB;          // bytes of one V tile
    static constexpr int kSwzMask = FP8 ? (kCpr >= 8 ? 7 : 3) : (kCpr >= 16 ? 7 : 3);
    static constexpr int kQStride = D + 8;             // bf16 per staged Q row
    static constexpr int kQBytes = kMfmaRows * kQStride * 2;
    static constexpr int kStage1 = kStage > kQBytes ? kStage : kQBytes;   // stage 1 doubles as Q staging
    static_assert(kCpr >= 4 && kCpr <= 64, "row must span 4..64 chunks");
    // chunk c of tile row k is stored at chunk c ^ swz(k): consecutive rows land on
    // distinct banks for the transpose reads (8 B per lane, 4 or 8 rows per group)
    static __device__ __forceinline__ int swz(int k) { return FP8 ? (k & kSwzMask) : ((k & kSwzMask) << 1); }
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

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt split over
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Source row for keys without a usable cache row (past the split's end, or in a
// block whose id is out of range): the DMA always issues, so every wave has the
// same number of loads in flight, and such keys read zeros (a bad block id
// poisons the key's score instead).
__device__ __attribute__((aligned(16))) const unsigned char kZeroRow[512] = {};

// One 16-byte-per-lane global -> LDS copy: lane l's 16 bytes land at lds_dst + 16 l
// (lds_dst uniform across the wave).  Written as inline assembly on purpose: the
// compiler then does not track it, so workgroup barriers do not drain these loads;
// every read of the destination is ordered by an explicit vmcnt wait and a barrier.
// M0 holds the LDS base; nothing else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, const void* lds_dst) {
    const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)LDS_PTR(void, lds_dst));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(a), "v"(src)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

template <int D, bool FP8, bool OUT_F32>
__global__ __launch_bounds__(kMfmaThreads, 2) void partition_mfma_kernel(PartitionParams p) {
    using G = Geo<D, FP8>;
    constexpr int KS = D / 32;                   // 32-dim k-steps of S^T = K Q^T (one K load each)
    constexpr int DC = D / 8;                    // 8-element chunks of a Q row
    constexpr int DTW = D / 64;                  // 16-column tiles per wave in phase C
    static_assert(G::kRowB <= (int)sizeof(kZeroRow), "zero row too short");

    __shared__ __attribute__((aligned(16))) unsigned char vst0[G::kStage];    // V tile, even tiles
    __shared__ __attribute__((aligned(16))) unsigned char vst1[G::kStage1];   // V tile, odd tiles; Q staging first
    __shared__ __attribute__((aligned(16))) float sbuf[kMfmaRows * kSStride];
    __shared__ __attribute__((aligned(16))) int rowidx[kMfmaMaxKeys];
    __shared__ int tbl[kMfmaThreads];
    __shared__ float alpha_s[kMfmaRows];
    __shared__ float st_m[kMfmaRows];
    __shared__ float st_l[kMfmaRows];
    uint16_t* qs = reinterpret_cast<uint16_t*>(vst1);

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

    // ---- Q rows of this chunk -> LDS (coalesced 16-byte loads, zero past R) ---------
    const uint16_t* qg = reinterpret_cast<const uint16_t*>(p.q);
    for (int item = tid; item < kMfmaRows * DC; item += kMfmaThreads) {
        const int row = item / DC, c = item - row * DC;
        const int r = rc * kMfmaRows + row;
        const bool rv = r < p.R;
        const int i = rv ? r / p.G : 0;
        const int h = g * p.G + (rv ? r - i * p.G : 0);
        const uint4 v = ld_global_16(qg + (((int64_t)b * p.n_q + i) * p.H + h) * D + c * 8);
        *reinterpret_cast<uint4*>(qs + row * G::kQStride + c * 8) = rv ? v : make_uint4(0, 0, 0, 0);
    }

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
    if (short_row) tbl[tid] = tb;

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
    __syncthreads();   // tbl and the Q rows are in LDS

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
    uint4 qreg[2][KS];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qreg[rt][ks] = *reinterpret_cast<const uint4*>(qs + (rt * 16 + l16) * G::kQStride + ks * 32 + q4 * 8);
    __syncthreads();   // rowidx ready; the Q staging area (V stage 1) is free again

    const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k);
    const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v);

    // K rows of tile t for this wave (A operand, key t*64 + wave*16 + l16), as stored:
    // KS loads per lane, converted to bf16 only when phase A uses them.
    using KRaw = typename std::conditional<FP8, uint2, uint4>::type;
    KRaw kraw[KS];
    auto load_k = [&](int t) {
        const int kri = rowidx[t * kT + wave * 16 + l16];
        const int64_t ke = (int64_t)max(kri, 0) * D + q4 * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (FP8)
                kraw[ks] = ld_global_8(kbase + ke + ks * 32);
            else
                kraw[ks] = ld_global_16(kbase + (ke + ks * 32) * 2);
        }
    };
    // V rows of tile t for this wave's 16 keys -> LDS stage, chunks swizzled by row:
    // exactly G::kNv DMA instructions per wave, whatever the keys are.
    auto dma_v = [&](int t, unsigned char* stage) {
#pragma unroll
        for (int ins = 0; ins < G::kNv; ++ins) {
            const int row0 = wave * 16 + ins * G::kRpi;            // first tile row of this instruction
            const int row = row0 + lane / G::kCpr;
            const int chunk = (lane % G::kCpr) ^ G::swz(row);
            const int ri = rowidx[t * kT + row];
            const unsigned char* src = ri >= 0 ? vbase + (int64_t)ri * G::kRowB + chunk * 16 : kZeroRow + chunk * 16;
            dma16(src, stage + row0 * G::kRowB);       // lane l lands at row0 * kRowB + 16 l
        }
    };

    float m_run = -INFINITY, l_run = 0.0f;   // phase-B lanes: row wave*8 + lane/8
    f32x4_t o[DTW][2];
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt) o[dt][0] = o[dt][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int brow = wave * 8 + (lane >> 3);
    const int bcol = (lane & 7) * 8;
    const int dbase = wave * DTW * 16;

    if (ntiles > 0) {
        dma_v(0, vst0);
        load_k(0);
    }
    // vcur holds V of tile t (its DMA was issued during tile t-1); V of tile t+1
    // goes to vnext.
    for (int t = 0; t < ntiles; ++t) {
        unsigned char* vcur = (t & 1) ? vst1 : vst0;
        unsigned char* vnext = (t & 1) ? vst0 : vst1;
        const bool more = t + 1 < ntiles;

        // ---- phase A: scores of this wave's 16 keys ------------------------------------
        // Keys without a cache row were loaded from row 0: their scores are masked
        // below (a select, so whatever row 0 holds cannot leak); a bad block id turns
        // the key's score into NaN.
        uint4 ka[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (FP8)
                ka[ks] = e4m3x8_to_bf16x8(kraw[ks]);
            else
                ka[ks] = kraw[ks];
        }
        const int4 kr4 = *reinterpret_cast<const int4*>(rowidx + t * kT + wave * 16 + q4 * 4);
        const int krs[4] = {kr4.x, kr4.y, kr4.z, kr4.w};
        float4 sv[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mfma_bf16(ka[ks], qreg[rt][ks], acc);
            // lane holds S^T[key t*64 + wave*16 + q4*4 + e][row rt*16 + l16]
            float* svp = reinterpret_cast<float*>(&sv[rt]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tt = t * kT + wave * 16 + q4 * 4 + e;
                const int j = k0 + tt;
                const bool ok = tt < nk && j >= row_lo[rt] && j <= row_hi[rt];
                const float sc = krs[e] == -1 ? __builtin_nanf("") : acc[e] * scale_log2;
                svp[e] = ok ? sc : -INFINITY;
            }
        }
        if (t > 0) __syncthreads();   // every wave has finished phase C of tile t-1 (it read P over S)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
            *reinterpret_cast<float4*>(sbuf + (rt * 16 + l16) * kSStride + wave * 16 + q4 * 4) = sv[rt];
        __syncthreads();

        // ---- phase B: next V tile streams in; running max / sum; P (hi, lo) over S -----
        if (more) {
            dma_v(t + 1, vnext);
            load_k(t + 1);
        }
        {
            float* srow = sbuf + brow * kSStride;
            const float4 a0 = *reinterpret_cast<const float4*>(srow + bcol);
            const float4 a1 = *reinterpret_cast<const float4*>(srow + bcol + 4);
            const float svb[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            float mt = svb[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) mt = fmaxf(mt, svb[e]);
            mt = max8(mt);
            const float m_new = fmaxf(m_run, mt);
            const float mu = m_new == -INFINITY ? 0.0f : m_new;
            const float alpha = exp2f(m_run - mu);
            float psum = 0.0f;
            uint32_t ph[4], pl[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const float p0 = exp2f(svb[2 * e2] - mu);
                const float p1 = exp2f(svb[2 * e2 + 1] - mu);
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
        // This wave's V rows of tile t have landed once at most the kNv V loads and KS
        // K loads of tile t+1, issued after them, are still in flight.
        if (more)
            wait_vmcnt<KS + G::kNv>();
        else
            wait_vmcnt<0>();
        __syncthreads();

        // ---- phase C: O^T = alpha O^T + V^T P^T over this tile ---------------------------
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
                    const int d0 = dbase + dt * 16;
                    uint4 a;
                    if constexpr (FP8) {
                        // lanes 2r + c of a 16-lane group read key 8*q4 + r, bytes d0 + 8c..+7;
                        // lane j receives column d0 + j of those 8 keys
                        const int kr = ks2 * 32 + q4 * 8 + (l16 >> 1);
                        const int d = d0 + 8 * (l16 & 1);
                        const int off = kr * G::kRowB + (((d >> 4) ^ G::swz(kr)) << 4) + (d & 15);
                        const int2_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(int2_t, vcur + off));
                        a = e4m3x8_to_bf16x8(make_uint2((uint32_t)w[0], (uint32_t)w[1]));
                    } else {
                        // lanes 4r + c read key base + r, columns d0 + 4c..+3; lane j receives
                        // column d0 + j of those 4 keys (two reads cover 8 keys)
                        uint32_t wv[4];
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const int kr = ks2 * 32 + q4 * 8 + hh * 4 + (l16 >> 2);
                            const int d = d0 + 4 * (l16 & 3);
                            const int off = kr * G::kRowB + (((d >> 3) ^ G::swz(kr)) << 4) + (d & 7) * 2;
                            const short4_t v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(short4_t, vcur + off));
                            wv[2 * hh] = (uint32_t)(uint16_t)v4[0] | ((uint32_t)(uint16_t)v4[1] << 16);
                            wv[2 * hh + 1] = (uint32_t)(uint16_t)v4[2] | ((uint32_t)(uint16_t)v4[3] << 16);
                        }
                        a = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                    }
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) {
                        o[dt][rt] = mfma_bf16(a, bh[rt], o[dt][rt]);
                        o[dt][rt] = mfma_bf16(a, bl[rt], o[dt][rt]);
                    }
                }
            }
        }
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
