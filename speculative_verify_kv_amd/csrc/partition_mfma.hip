// Split-KV partition kernel on gfx950 matrix cores (bf16 MFMA 16x16x32).
//
// One workgroup owns one (problem b, KV head g, row chunk, column split, KV split
// s).  A KV head's query rows are its n_q queries times the H/Hkv heads that share
// it (row r = i * G + head-in-group), so a verify step with n_q = 8 and GQA 4 is
// one dense 32-row tile.  Launches that leave most CUs idle take 16-row chunks,
// each run by two or four workgroups that split the output columns (all load every
// K row and compute the same scores; each loads its part of every V row); launches
// with many rows per KV head take 64-row chunks, so that each K/V tile serves more
// rows.  The split's keys are walked in tiles of 64 (or 32) through an LDS ring
// filled by direct global-to-LDS loads (non-temporal where two workgroups share a CU).
//
// With 64-key tiles, compute wave w owns 16 query rows (a row block), one 32-key
// half of every tile's keys, with an online softmax of its own, and a set of the
// workgroup's output columns: all of them when two workgroups fit in a CU's LDS or
// the chunk has 64 rows, half of them otherwise (so that a SIMD still runs two
// waves).  With 32-key tiles every wave takes all keys of its row block; in 32-row
// chunks the waves split the columns, in 64-row chunks each wave has all of them.
// 16-row workgroups add as many loader waves, which only load and pass barriers.
// Per tile:
//   S^T = K . Q^T        matrix cores; K rows from LDS, Q^T in registers for the
//                        whole call; window (t - W, t] mask and scale applied
//   softmax              in registers: row max and sum across the four 16-lane
//                        groups with lane-swap permutes; P = 2^(S - max) as two
//                        bf16 terms (hi + lo) for bfloat16 caches, one for E4M3
//   O^T += V^T . P^T     matrix cores; P^T straight from registers, V^T from the
//                        row-major V tile by LDS transpose reads
// The ring has two stages (four where they are small).  While the waves work on
// tile t, each issues its share of the loads of the tile NS-1 ahead into the stage
// that tile t-1 held, between the score matrix ops.  One barrier per tile hands a
// landed stage to all waves and frees the stage of tile t-1.  At the end the two
// key halves of each row block merge their (max, sum, O) through LDS.
//
// Cache rows sit in LDS with their 16-byte chunks XOR-swizzled by row so that
// the matrix-operand reads of consecutive keys hit distinct LDS banks.  Keys
// past the split's end read a zero row; keys in a block whose id is out of range
// read a NaN K row and a zero V row, which makes their score NaN wherever the
// window covers them.  The workgroup writes the final output (S == 1) or a
// normalised partial and its log2-sum-exp for the merge kernel (S > 1).
//
// Semantics follow "The Fast Gemma Challenge: our verified-SOTA recipe, in full"
// (manifest: SLIDING_WINDOW, SPECULATIVE_CONFIG, SPLITKV_VERIFY,
// SPLITKV_VERIFY_MAX_Q; "What each piece does, and why"): each query attends to
// the most recent W positions up to its own, the target and drafts of one step
// are scored together, and a long KV range is split across workgroups.

#include <hip/hip_runtime.h>

#include "kv_access.h"
#include "split_merge.h"
#include "swattn_internal.h"

namespace swattn {
namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef int int2_t __attribute__((ext_vector_type(2)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// KT = keys per tile.  64: two key halves of 32, one per wave pair, merged at the
// end.  32: every wave takes all 32 keys of a tile and the waves split the output
// columns instead, which halves the LDS a workgroup needs (no merge either).
template <int D, bool FP8, int KT, int RB = 2, int CS = 1>
struct Geo {
    static constexpr int kT = KT;
    static constexpr bool kSplitKeys = KT == 64;
    static_assert(KT == 32 || KT == 64, "tiles of 32 or 64 keys");
    static constexpr int kElt = FP8 ? 1 : 2;
    static constexpr int kRowB = D * kElt;                  // bytes per cache row
    static constexpr int kCpr = kRowB / 16;                 // 16-byte chunks per row
    static constexpr int kRpi = 64 / kCpr;                  // rows per 64-lane load instruction (1 KiB)
    static constexpr int kNiK = kT / kRpi;                  // load instructions per K (or V) tile
    static constexpr int kTileB = kT * kRowB;               // bytes of one K tile
    static_assert(kCpr >= 4 && kCpr <= 64 && kNiK * 1024 == kTileB, "tile geometry");
    // Row chunks may also split the output columns between two or four workgroups: each
    // loads whole K rows (all compute the chunk's scores) and its own part of every V
    // row.
    static_assert(CS == 1 || ((CS == 2 || CS == 4) && KT == 64), "column splits with 64-key tiles only");
    static constexpr int kCS = CS;                          // column splits
    static constexpr int kRowBV = kRowB / kCS;              // bytes of a V row this workgroup loads
    static constexpr int kCprV = kRowBV / 16;
    static constexpr int kRpiV = 64 / kCprV;
    static constexpr int kNiV = kT / kRpiV;                 // load instructions per V tile
    static constexpr int kTileBV = kT * kRowBV;
    static_assert(kCprV >= 4 && kNiV * 1024 == kTileBV, "V tile geometry");
    static constexpr int kStageB = kTileB + kTileBV;
    // Q rows of the chunk, staged once per workgroup in LDS (bfloat16, kRows x D):
    // every compute wave reads its Q^T operand from there.  64-row chunks with 32-key
    // tiles do without: each of their four waves owns one row block and loads its Q^T
    // operand straight into registers.
    static constexpr bool kQLds = RB != 4 || KT == 64;
    static constexpr int kRowQ = D * 2;
    static constexpr int kCprQ = kRowQ / 16;
    static constexpr int kQB = kQLds ? 16 * RB * kRowQ : 0;
    static constexpr int kNiQ = kQB / 1024;                 // load instructions of the Q rows
    static_assert(kNiQ * 1024 == kQB, "Q geometry");
    // Stages of the K/V ring (the ring plus < 14 KiB of tables per workgroup, 160 KiB
    // of LDS per CU): four where two workgroups per CU still fit with them (up to three
    // tiles in flight absorb the tail latency of a loaded memory system), else two.
    // (A CU's load rate, about 30-45 GB/s, bounds these chains: rings that request
    // every tile of a chunk up front measured slower, since tile 0 then lands later.)
    static constexpr int kNS = 2 * (4 * kStageB + 14 * 1024) <= 160 * 1024 ? 4 : 2;
    // Workgroups per CU that the LDS allows.  Where only one fits, the workgroup has 8
    // waves (32-row chunks split the output columns across two wave sets, 64-row chunks
    // have four row blocks) so that every SIMD still holds two waves; otherwise it has
    // 4 waves.  Either way a SIMD runs two waves, so each may hold 256 registers.
    static constexpr int kBlocks = 2 * (kNS * kStageB + 14 * 1024) <= 160 * 1024 ? 2 : 1;
    // Where two workgroups share a CU, and in 64-row chunks (whose 32 KiB of Q rows would
    // not fit beside the ring), the prologue leaves the last ring stage free (its tile goes
    // out with tile 0's scores): Q is staged there.  Otherwise it has a region of its own.
    static constexpr bool kQAlias = kQLds && (kBlocks == 2 || RB == 4);
    static_assert(!kQAlias || kTileB >= kQB, "Q fits the K part of a ring stage");
    static_assert(kQAlias || kNS * kStageB + 14 * 1024 + kQB <= 160 * 1024, "one workgroup's LDS");
    // column sets: 64-key tiles split them only where one workgroup fills the CU;
    // 32-key tiles split them in two (their waves do not split the keys), except in
    // 64-row chunks, whose four waves take one row block each
    static constexpr int kND = RB == 4 ? 1 : (kSplitKeys ? (kBlocks == 2 ? 1 : 2) : 2);
    // row blocks of 16 query rows per workgroup: 2; 1 for launches that leave most CUs
    // idle (two workgroups then share a 32-row chunk's keys, each with half the work); 4
    // for chunks of many query rows, so that every K/V tile serves 64 rows
    static_assert(RB == 2 || (RB == 1 && KT == 64) || (RB == 4 && CS == 1 && !FP8),
                  "16-row chunks with 64-key tiles; 64-row chunks for bfloat16 caches");
    static constexpr int kRows = 16 * RB;
    static constexpr int kLgRB = RB == 4 ? 2 : RB - 1;      // log2 of the row blocks
    static constexpr int kNWc = kSplitKeys ? 2 * RB * kND : RB * kND;   // compute waves: row blocks x key halves x column sets
    // 16-row workgroups (one per CU for bfloat16) add as many loader waves, which take
    // their share of every tile's loads and do no arithmetic: a workgroup's load rate
    // grows with the number of waves issuing its loads (a memory-only probe of the
    // verify step's 147 KB per workgroup: 10.5 us with 4 waves, 8.2 us with 8; the
    // verify step itself: 9.7 -> 8.7 us warm, cold unchanged).
    static constexpr int kNL = RB == 1 ? kNWc : 0;
    // Where two workgroups share a CU, their K/V and Q copies carry the non-temporal cache
    // policy: batched bf16 27.5 -> 24.7 us, batched E4M3 20.0 -> 18.9 us, full context
    // 4096 (32-key tiles) 48.2 -> 42.7 us.  Not in 64-row chunks, whose workgroups re-read
    // a unit's window from L2 (prefill of 512 positions 67.8 -> 69.9 us with it), nor at
    // one workgroup per CU, where it measured within +-1 us (verify, decode, full context
    // 1024 and 2048).
    static constexpr bool kStream = kBlocks == 2 && RB != 4;
    static constexpr int kNW = kNWc + kNL;
    static constexpr int kNT = kNW * 64;
    static constexpr int kShare = (kNiK + kNiV) / kNW;      // load instructions per wave per tile
    static_assert(kShare * kNW == kNiK + kNiV && kShare <= 16, "loads split evenly over the waves");
    static_assert(kNS >= 2 && kNS <= 4, "ring of 2 to 4 stages");
    static_assert(kNS * kShare < 64, "a wave's loads in flight must fit the vmcnt counter");
    // K rows: chunk c of row k is stored at c ^ swz_k(k); 16 consecutive rows (the
    // 16 lanes of an A-operand read) land on distinct bank groups.
    static __device__ __forceinline__ int swz_k(int k) { return k & (kCpr >= 16 ? 15 : kCpr - 1); }
    // Q rows: the same scheme for the B-operand reads of 16 consecutive rows
    static __device__ __forceinline__ int swz_q(int r) { return r & (kCprQ >= 16 ? 15 : kCprQ - 1); }
    // V rows (this workgroup's part of them).  The LDS serves a 64-bit transpose read 32
    // lanes at a time; those lanes must land on 16 distinct 16-byte chunks.  E4M3: lanes
    // 0-31 read one column chunk of keys {0..7, 16..23} of the 32-key half (lanes 32-63
    // keys {8..15, 24..31}), so the swizzle takes key bits 0-2 and 4.  bfloat16: lanes
    // 0-31 read two adjacent chunks of keys 0..7 of a 16-key group, so the swizzle (an
    // even chunk offset) takes key bits 0-2.  Measured: no bank conflicts left in the
    // bfloat16 kernels (21% of LDS-active cycles before), E4M3 38% -> 29%.
    static __device__ __forceinline__ int swz_v(int k) {
        if constexpr (FP8)
            return kCprV >= 16 ? ((k & 7) | (((k >> 4) & 1) << 3)) : (((k & 3) | ((k >> 2) & 4)) & (kCprV >= 8 ? 7 : 3));
        else
            return (((k & 3) << 1) | (((k >> 2) & 1) << 3)) & (kCprV - 1);
    }
};

// Source rows for keys without a usable cache row: zeros (past the split's end)
// and all-ones bytes, which are NaN both as bfloat16 and as E4M3 (bad block id).
struct FilledRow {
    uint32_t w[128];
    constexpr explicit FilledRow(uint32_t v) : w() {
        for (int i = 0; i < 128; ++i) w[i] = v;
    }
};
__device__ __attribute__((aligned(16))) const FilledRow kZeroRow(0u);
__device__ __attribute__((aligned(16))) const FilledRow kNanRow(0xFFFFFFFFu);

__device__ __forceinline__ f32x4_t mfma_bf16(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane groups holding one score
// row), every lane receiving the result.  Each swap returns the value and its partner's
// in some order; the max does not care which.
__device__ __forceinline__ float xgroup_max(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// 2^x by the hardware instruction alone.  Its arguments here are at most 8 (scores
// minus a running max, or a max difference); results below the normal range
// flush to zero, which no sum of these weights can register.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// kh ? a : b for two accumulator tiles.  The values pass through an empty asm
// first: otherwise the compiler turns the select of two array elements into a
// load from a selected address, and that runtime index moves the whole
// accumulator array to scratch memory.
__device__ __forceinline__ f32x4_t pick(bool first, f32x4_t a, f32x4_t b) {
    asm volatile("" : "+v"(a), "+v"(b));
    return first ? a : b;
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt split over
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The LDS address of an element of a __shared__ array, as a 32-bit offset.  Written for
// direct array elements only: the destination of a copy is chosen between these offsets,
// never between generic pointers into different LDS arrays (whose cast back to the LDS
// address space the compiler lowers with an illegal instruction).
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
    return (uint32_t)(uintptr_t)LDS_PTR(const void, p);
}

// One 16-byte-per-lane global -> LDS copy: lane l's 16 bytes land at LDS address
// lds_dst + 16 l (lds_dst uniform across the wave).  Written as inline assembly on purpose: the
// compiler then neither tracks it (workgroup barriers do not drain these loads)
// nor treats it as touching memory (LDS reads of the other stage move freely
// around it); it stays ordered with barriers and waits, which have side effects.
// Every read of the destination is ordered by an explicit vmcnt wait in the
// issuing wave and a barrier.  M0 holds the LDS base; nothing else in these
// kernels uses M0.  NT sets the non-temporal cache policy (a hint: the bytes read are
// the same).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_dst) {
    const uint32_t a = __builtin_amdgcn_readfirstlane(lds_dst);
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(a), "v"(src) : "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(a), "v"(src) : "m0");
}
#pragma clang diagnostic pop

template <int D, bool FP8, bool OUT_F32, int KT, int RB, int CS>
__global__ __launch_bounds__((Geo<D, FP8, KT, RB, CS>::kNT), (Geo<D, FP8, KT, RB, CS>::kBlocks)) void partition_mfma_kernel(PartitionParams p) {
    using G = Geo<D, FP8, KT, RB, CS>;
    constexpr int kT = KT;
    constexpr int NT = G::kNT;
    constexpr int KS = D / 32;                   // 32-dim k-steps of S^T = K Q^T
    constexpr int DC = D / G::kCS;               // output columns of this workgroup
    constexpr int DH = DC / G::kND;              // output columns of one wave set
    constexpr int DB = DH / 16;                  // 16-column output tiles per wave
    constexpr int SH = G::kShare;                // this wave's loads per tile
    // P enters the PV product as one bfloat16 term for E4M3 caches (its rounding,
    // below 2^-9 relative, is far inside what 8-bit values carry) and as two terms
    // (hi + lo, about 16 bits) for bfloat16 caches, whose outputs are held to 2e-3.
    constexpr bool kSingleP = FP8;

    constexpr int NS = G::kNS;
    __shared__ __attribute__((aligned(16))) unsigned char kst[NS][G::kTileB];
    __shared__ __attribute__((aligned(16))) unsigned char vst[NS][G::kTileBV];
    // source of every key's K and V row (a cache row, the zero row or the NaN row)
    __shared__ __attribute__((aligned(16))) const unsigned char* kptr[kMfmaMaxKeys];
    __shared__ __attribute__((aligned(16))) const unsigned char* vptr[kMfmaMaxKeys];
    __shared__ int tbl[NT];
    __shared__ float xstat[RB == 4 ? 4 : 2][2][2][16];   // [rb][kh][m, l][row]
    // the chunk's Q rows: the K part of the last ring stage where two workgroups share a
    // CU, else a region of their own (none for 64-row chunks: their Q goes to registers)
    __shared__ __attribute__((aligned(16))) unsigned char qst[G::kQAlias || !G::kQLds ? 16 : G::kQB];
    static_assert(!G::kSplitKeys || RB * 2 * G::kND * 16 * (D / G::kCS / G::kND / 2) * 4 <= (int)sizeof(kst),
                  "merge exchange fits in the K stages");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool loader = G::kNL > 0 && wave >= G::kNWc;   // loads and barriers only
    const int cw = loader ? 0 : wave;            // compute-wave index (loaders mirror wave 0)
    const int l16 = lane & 15;
    const int q4 = lane >> 4;
    const int rb = RB == 4 ? cw & 3 : (RB == 2 ? cw & 1 : 0);   // 16-row block
    // key half of every tile (64-key tiles) and column set
    const int kh = G::kSplitKeys ? (cw >> G::kLgRB) & 1 : 0;
    const int dh = G::kSplitKeys ? cw >> (G::kLgRB + 1) : (RB == 4 ? 0 : (cw >> 1) & 1);

    // grid (B * Hkv, row chunks x column splits, splits)
    const int s = blockIdx.z;
    const int rc = blockIdx.y / G::kCS;
    const int cs = blockIdx.y - rc * G::kCS;     // this workgroup's columns: cs*DC .. +DC-1
    const int g = blockIdx.x % p.Hkv;
    const int b = blockIdx.x / p.Hkv;

    // The chunk's Q rows go into LDS at once, once per workgroup, each wave issuing a
    // share (waves of every role: with the loader waves alone issuing them, the E4M3
    // 16-row kernel needs more registers than two waves per SIMD allow); a row past R
    // loads a valid row.  They land while ctx_len and the block table are fetched and
    // are waited for before the block-table barrier, so the compute waves read their
    // Q^T operands from LDS without a barrier of their own, and no tile competes with
    // them for the CU's load rate.
#pragma unroll
    for (int jj = 0; jj < (G::kNiQ + G::kNW - 1) / G::kNW; ++jj) {
        const int j = wave + jj * G::kNW;                            // wave-uniform
        if (j < G::kNiQ) {
            const int slot = j * 64 + lane;
            const int row = slot / G::kCprQ, pc = slot % G::kCprQ;
            const int r = min(rc * G::kRows + row, p.R - 1);
            const int i = r / p.G, h = g * p.G + (r - i * p.G);
            const unsigned char* src = reinterpret_cast<const unsigned char*>(p.q) +
                                       (((int64_t)b * p.n_q + i) * p.H + h) * G::kRowQ + ((pc ^ G::swz_q(row)) << 4);
            if constexpr (G::kQAlias)
                dma16<G::kStream>(src, lds_addr(&kst[NS - 1][j * 1024]));
            else
                dma16<G::kStream>(src, lds_addr(&qst[j * 1024]));
        }
    }

    // A block-table row that fits one entry per thread is read while ctx_len is in
    // flight, which removes one dependent round trip to memory.
    const bool short_row = p.max_blocks <= NT;
    const int tb = (short_row && tid < p.max_blocks) ? p.block_table[(int64_t)b * p.max_blocks + tid] : 0;

    // this lane's query row (row rb*16 + l16 of the chunk); a row past R has an empty
    // window and is never written
    const int qrow = rc * G::kRows + rb * 16 + l16;
    const bool qvalid = qrow < p.R;
    const int qi = qvalid ? qrow / p.G : 0;
    // Q^T operand of this lane: row rb*16 + l16 of the chunk, dims ks*32 + q4*8 .. +7.
    // 64-row chunks load it here, beside the ctx_len and block-table round trip (a row
    // past R loads a valid row); the others read it from the Q rows in LDS below.
    uint4 qreg[KS];
    if constexpr (!G::kQLds) {
        const int r = min(qrow, p.R - 1);
        const int i = r / p.G, h = g * p.G + (r - i * p.G);
        const uint4* qp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.q) +
                                                         (((int64_t)b * p.n_q + i) * p.H + h) * D + q4 * 8);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[ks] = qp[ks * 4];
    }
    float scale_log2 = p.scale_log2;
    float out_scale = 1.0f;
    if constexpr (FP8) {
        scale_log2 *= p.k_scale[g];
        out_scale = p.v_scale[g];
    }

    const int ctx = p.ctx_len[b];
    const bool seq_ok = ctx >= p.n_q && ctx <= p.max_blocks * p.bs && ctx <= p.max_ctx;
    const int pos0 = seq_ok ? ctx - p.n_q : 0;             // position of query 0
    // The chunk's keys: the union of its rows' windows, queries qi_lo .. qi_hi, i.e.
    // positions [pos0 + qi_lo - W + 1, pos0 + qi_hi]; the split takes a 1/S share.
    const int qi_lo = rc * G::kRows / p.G;
    const int qi_hi = min(p.R - 1, rc * G::kRows + G::kRows - 1) / p.G;
    const int u_lo = max(0, pos0 + qi_lo - p.window + 1);
    const int u_hi = pos0 + qi_hi + 1;                     // one past the last key
    int k0 = 0, nk = 0;
    if (seq_ok) {
        const int kps = (u_hi - u_lo + p.S - 1) / p.S;
        k0 = u_lo + s * kps;
        nk = max(0, min(u_hi, k0 + kps) - k0);             // <= kMfmaMaxKeys by the plan
    }
    const int ntiles = (nk + kT - 1) / kT;
    if (short_row) tbl[tid] = tb;
    wait_vmcnt<0>();   // this wave's share of the Q rows has landed too
    __syncthreads();   // tbl and the Q rows are in LDS

    // ---- key -> source rows: cache row (phys * Hkv + g) * bs + off of K and V; keys
    //      past the split read the zero row, keys in a bad block a NaN K and zero V row
    {
        const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k);
        const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v);
        const unsigned char* zrow = reinterpret_cast<const unsigned char*>(&kZeroRow);
        const unsigned char* nrow = reinterpret_cast<const unsigned char*>(&kNanRow);
        for (int t = tid; t < ntiles * kT; t += NT) {
            const unsigned char* kp = zrow;
            const unsigned char* vp = zrow;
            if (t < nk) {
                const int j = k0 + t;
                const int blk = p.bs_log2 >= 0 ? j >> p.bs_log2 : j / p.bs;
                const int off = j - blk * p.bs;
                const int phys = short_row ? tbl[blk] : p.block_table[(int64_t)b * p.max_blocks + blk];
                if (phys >= 0 && phys < p.num_blocks) {
                    const int64_t rowb = ((int64_t)(phys * p.Hkv + g) * p.bs + off) * G::kRowB;
                    kp = kbase + rowb;
                    vp = vbase + rowb;
                    // a new row (fused append, bfloat16 only): from the caller's buffer
                    if (!FP8 && p.k_new != nullptr && j >= pos0) {
                        const int64_t nrow = (((int64_t)b * p.n_q + (j - pos0)) * p.Hkv + g) * G::kRowB;
                        kp = reinterpret_cast<const unsigned char*>(p.k_new) + nrow;
                        vp = reinterpret_cast<const unsigned char*>(p.v_new) + nrow;
                    }
                } else {
                    kp = nrow;
                }
            }
            kptr[t] = kp;
            vptr[t] = vp;
        }
    }
    __syncthreads();   // source tables ready

    // ---- this wave's loads of a tile (kNiK K and kNiV V instructions; K instruction i
    //      fills rows i*kRpi .. +kRpi-1, lane l of it chunk l % kCpr of row i*kRpi + l/kCpr,
    //      V likewise).  Without loader waves every wave takes an equal share of each kind:
    //      K instructions wave*SHK .. +SHK-1 as its loads 0 .. SHK-1, then V instructions
    //      wave*SHV .. +SHV-1, so that whether a load is K or V is known at compile time and
    //      its table entry is a fixed offset from one address per tile (prefill 64.8 ->
    //      62.3 us).  With loader waves, instructions wave*SH .. +SH-1 of the K-then-V list:
    //      the compute waves then issue K loads only (verify and decode measured slower
    //      with the even split).
    constexpr bool kEven = G::kNL == 0;
    constexpr int SHK = kEven ? G::kNiK / G::kNW : 0;
    constexpr int SHV = kEven ? G::kNiV / G::kNW : 0;
    static_assert(!kEven || (SHK * G::kNW == G::kNiK && SHV * G::kNW == G::kNiV && SHK + SHV == SH),
                  "every wave takes an equal share of the K and of the V instructions");
    const int rsub = lane / G::kCpr;
    const int pch = lane % G::kCpr;              // LDS chunk this lane fills (K)
    const int rsub_v = lane / G::kCprV;
    const int pch_v = lane % G::kCprV;           // (V)
    // captures by value: a by-reference closure pins the captured locals in scratch
    auto rows_of = [=](int t, const unsigned char** src) __attribute__((always_inline)) {   // this wave's SH source rows of tile t
#pragma unroll
        for (int j = 0; j < SH; ++j) {
            const int insk = kEven ? wave * SHK + j : wave * SH + j;                  // as K
            const int insv = kEven ? wave * SHV + j - SHK : wave * SH + j - G::kNiK;  // as V
            if (kEven ? j >= SHK : insk >= G::kNiK) {
                const int row = insv * G::kRpiV + rsub_v;
                src[j] = vptr[t * kT + row] + cs * G::kRowBV + ((pch_v ^ G::swz_v(row)) << 4);
            } else {
                const int row = insk * G::kRpi + rsub;
                src[j] = kptr[t * kT + row] + ((pch ^ G::swz_k(row)) << 4);
            }
        }
    };
    // LDS slot of this wave's load j of a tile in stage st
    auto slot_of = [=](int st, int j) __attribute__((always_inline)) {
        if constexpr (kEven)
            return j >= SHK ? lds_addr(&vst[st][(wave * SHV + j - SHK) * 1024]) : lds_addr(&kst[st][(wave * SHK + j) * 1024]);
        const int ins = wave * SH + j;
        return ins >= G::kNiK ? lds_addr(&vst[st][(ins - G::kNiK) * 1024]) : lds_addr(&kst[st][ins * 1024]);
    };
    // loads j0 .. j1-1 of this wave's share of tile t
    auto issue_range = [=](int t, int j0, int j1) __attribute__((always_inline)) {
        const unsigned char* src[SH];
        rows_of(t, src);
#pragma unroll
        for (int j = 0; j < SH; ++j) {
            if (j < j0 || j >= j1) continue;
            dma16<G::kStream>(src[j], slot_of(t % NS, j));
        }
    };

    const int row_lo = qvalid ? max(0, pos0 + qi - p.window + 1) : 1;
    const int row_hi = qvalid ? pos0 + qi : 0;
    // key t of the split (position k0 + t) counts for this row iff k0 + t - row_lo, as an
    // unsigned number, is below row_cnt: the row's window cut at the split's last key
    const int row_cnt = max(0, min(row_hi, k0 + nk - 1) - row_lo + 1);

    // The compiler cannot see the loads below, so a wait of its own for an earlier
    // load would count them as older: nothing it issued is left in flight from here.
    wait_vmcnt<0>();
    // The first tiles go out together, one per stage: all NS where one workgroup has
    // the CU, NS-1 where two share it (tile NS-1 then goes out with tile 0's scores:
    // a wave whose loads stall at issue reaches its first tile sooner; batched E4M3,
    // 512 workgroups: 21.4 -> 20.2 us) or where Q sits in the last stage.
    constexpr int kPro = (G::kQAlias || G::kBlocks == 2) ? NS - 1 : NS;
#pragma unroll
    for (int t = 0; t < kPro; ++t)
        if (t < ntiles) issue_range(t, 0, SH);

    // The Q^T operands from the Q rows in LDS (landed before the block-table barrier).
    // The barrier of tile 0 orders these reads before tile NS-1 goes into the stage that
    // Q may share.
    if constexpr (G::kQLds) {
        if (ntiles > 0 && !loader) {
            const int row = rb * 16 + l16;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int off = row * G::kRowQ + (((ks * 4 + q4) ^ G::swz_q(row)) << 4);
                if constexpr (G::kQAlias)
                    qreg[ks] = *reinterpret_cast<const uint4*>(&kst[NS - 1][off]);
                else
                    qreg[ks] = *reinterpret_cast<const uint4*>(&qst[off]);
            }
        }
    }
    float m_run = -INFINITY, l_run = 0.0f;   // row l16 of block rb, keys of half kh
    // The row sum of P accumulates on the matrix cores beside O^T: a matrix op with an
    // all-ones A operand gives every lane its row's sum of the tile's (rounded) P terms, and
    // the accumulator is rescaled with O^T.  That replaces eight adds and a cross-lane
    // reduction per tile with one or two matrix ops, and the weights are normalised by the
    // sum of exactly the terms that entered the PV product.
    f32x4_t lacc = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint4 kOnes = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);   // bf16 1.0
    f32x4_t o[DB];                           // lane holds O^T[dcol0 + db*16 + 4*q4 + e][row l16]
    const int dcol0 = dh * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int kbase_t = kh * 32;             // this wave's keys within a tile (32 of them)

    for (int t = 0; t < ntiles; ++t) {
        // This wave's loads of tile t have landed once only those of younger tiles are
        // pending: tiles t+1 .. t+ahead, issued before this point.
        const int ahead = min(t == 0 ? kPro - 1 : NS - 2, ntiles - 1 - t);
        switch (ahead) {
            case 0: wait_vmcnt<0>(); break;
            case 1: wait_vmcnt<SH>(); break;
            case 2: wait_vmcnt<2 * SH>(); break;
            default: wait_vmcnt<3 * SH>(); break;
        }
        __syncthreads();   // B_t: tile t is in its stage for every wave; tile t-1's stage is free
        const int tn = t + NS - 1;                         // goes into tile t-1's stage
        const bool prefetch = t >= kPro - (NS - 1) && tn < ntiles;
        // This wave's loads of tile tn go out between the matrix ops of the scores
        // below: a load instruction can stall its wave at issue while the memory
        // pipeline is busy, and the matrix ops already issued keep running meanwhile.
        const unsigned char* src[SH];
        if (prefetch) rows_of(tn, src);
        auto load_one = [=](int j, const unsigned char* from) __attribute__((always_inline)) {
            dma16<G::kStream>(from, slot_of(tn % NS, j));
        };
        if (loader) {
            if (prefetch) {
#pragma unroll
                for (int j = 0; j < SH; ++j) load_one(j, src[j]);
            }
            continue;
        }
        constexpr int kPerStep = (SH + KS - 1) / KS;        // loads after each k-step's matrix ops
        const unsigned char* kc = kst[t % NS];
        const unsigned char* vc = vst[t % NS];
        // a key half wholly past the split's end (the tail of the last tile) adds nothing
        const int key_lo = t * kT + kbase_t;                // this wave's first key of the tile
        if (key_lo >= nk) {
            if (prefetch) {
#pragma unroll
                for (int j = 0; j < SH; ++j) load_one(j, src[j]);
            }
            continue;
        }
        // all 32 keys inside every row's window and the split: no mask needed
        const bool inside = key_lo + 31 < nk && k0 + key_lo >= row_lo && k0 + key_lo + 31 <= row_hi;
        const bool unmasked = __builtin_amdgcn_ballot_w64(!inside) == 0;

        // ---- scores: lane holds S[row l16][key kbase_t + kb*16 + 4*q4 + e] -------------
        float sv[2][4];
        {
        // Every K operand of the tile is read first; the two key blocks then run as
        // independent accumulation chains, interleaved.
        uint4 ka[2][KS];                         // E4M3: 8 bytes in .x/.y, converted at use
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int krow = kbase_t + kb * 16 + l16;
            const unsigned char* kr = kc + krow * G::kRowB;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (FP8) {
                    const int c = ks * 2 + (q4 >> 1);
                    const uint2 w =
                        *reinterpret_cast<const uint2*>(kr + ((c ^ G::swz_k(krow)) << 4) + (q4 & 1) * 8);
                    ka[kb][ks] = make_uint4(w.x, w.y, 0u, 0u);
                } else {
                    const int c = ks * 4 + q4;
                    ka[kb][ks] = *reinterpret_cast<const uint4*>(kr + ((c ^ G::swz_k(krow)) << 4));
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the matrix ops
        f32x4_t sacc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                uint4 a = ka[kb][ks];
                if constexpr (FP8) a = e4m3x8_to_bf16x8(make_uint2(a.x, a.y));
                sacc[kb] = mfma_bf16(a, qreg[ks], sacc[kb]);
            }
            if (prefetch) {
#pragma unroll
                for (int j = ks * kPerStep; j < (ks + 1) * kPerStep && j < SH; ++j) load_one(j, src[j]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const f32x4_t acc = sacc[kb];
            if (unmasked) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[kb][e] = acc[e] * scale_log2;
            } else {
                const int d0 = k0 + key_lo + kb * 16 + q4 * 4 - row_lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = (uint32_t)(d0 + e) < (uint32_t)row_cnt;
                    sv[kb][e] = ok ? acc[e] * scale_log2 : -INFINITY;
                }
            }
        }

        }   // scores

        // ---- online softmax in registers --------------------------------------------
        // The running max m_run only moves when a row's tile max exceeds it by more than
        // 2^8: P = 2^(S - m_run) stays below 256, and the rescale of O^T (a multiply per
        // accumulator) is skipped on every tile where no row of the wave moves.  The
        // result is the same softmax: O^T and the sum carry the same reference max.
        float mt = sv[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) mt = fmaxf(mt, sv[kb][e]);
        mt = xgroup_max(mt);
        const bool grow = mt > m_run + 8.0f;                // never for a row with no key yet
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float m_new = grow ? mt : m_run;
            const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.0f : m_new));
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = o[db] * alpha;
            lacc = lacc * alpha;
            m_run = m_new;
        }
        const float mu = m_run == -INFINITY ? 0.0f : m_run;
        // B operand of the PV step: k-slot hh*4 + e <-> key kbase_t + hh*16 + 4*q4 + e
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                const float p0 = fast_exp2(sv[hh][2 * e2] - mu);
                const float p1 = fast_exp2(sv[hh][2 * e2 + 1] - mu);
                const uint32_t hp = pack_bf16x2(p0, p1);
                wh[hh * 2 + e2] = hp;
                if constexpr (!kSingleP) {
                    // the residuals against the rounded pair, unpacked in place
                    wl[hh * 2 + e2] = pack_bf16x2(p0 - __uint_as_float(hp << 16), p1 - __uint_as_float(hp & 0xFFFF0000u));
                } else {
                    wl[hh * 2 + e2] = 0u;
                }
            }
        }
        const uint4 ph = make_uint4(wh[0], wh[1], wh[2], wh[3]);
        const uint4 pl = make_uint4(wl[0], wl[1], wl[2], wl[3]);

        // ---- O^T = alpha O^T + V^T P^T ----------------------------------------------
        // Software-pipelined by hand: the V^T reads of step db+1 go out before the
        // matrix ops of step db.
        auto load_vt = [=](int db) __attribute__((always_inline)) {
            const int d0 = dcol0 + db * 16;
            uint4 a;
            if constexpr (FP8) {
                // lanes 2r + c read key kbase_t + (r & 3) + 4*q4 + 16*(r >> 2), bytes d0 + 8c..+7;
                // lane j receives column d0 + j of those 8 keys, k-slot r
                const int r = l16 >> 1;
                const int kr = kbase_t + (r & 3) + q4 * 4 + (r >> 2) * 16;
                const int d = d0 + 8 * (l16 & 1);
                const int off = kr * G::kRowBV + (((d >> 4) ^ G::swz_v(kr)) << 4) + (d & 15);
                const int2_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(int2_t, vc + off));
                a = make_uint4((uint32_t)w[0], (uint32_t)w[1], 0u, 0u);   // converted at use
            } else {
                // lanes 4r + c read key kbase_t + hh*16 + 4*q4 + r, columns d0 + 4c..+3; lane j
                // receives column d0 + j of those 4 keys, k-slots hh*4 + r
                uint32_t wv[4];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int kr = kbase_t + hh * 16 + q4 * 4 + (l16 >> 2);
                    const int d = d0 + 4 * (l16 & 3);
                    const int off = kr * G::kRowBV + (((d >> 3) ^ G::swz_v(kr)) << 4) + (d & 7) * 2;
                    const short4_t v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(short4_t, vc + off));
                    wv[2 * hh] = (uint32_t)(uint16_t)v4[0] | ((uint32_t)(uint16_t)v4[1] << 16);
                    wv[2 * hh + 1] = (uint32_t)(uint16_t)v4[2] | ((uint32_t)(uint16_t)v4[3] << 16);
                }
                a = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
            return a;
        };
        // every V^T operand first, then one matrix op per accumulator for the hi term
        // and one more for the lo term, so that consecutive ops are independent
        uint4 va[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) va[db] = load_vt(db);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            if constexpr (FP8) va[db] = e4m3x8_to_bf16x8(make_uint2(va[db].x, va[db].y));
            o[db] = mfma_bf16(va[db], ph, o[db]);
        }
        if constexpr (!kSingleP) {
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = mfma_bf16(va[db], pl, o[db]);
        }
        lacc = mfma_bf16(kOnes, ph, lacc);
        if constexpr (!kSingleP) lacc = mfma_bf16(kOnes, pl, lacc);
    }
    l_run = lacc[0];                             // every element holds row l16's sum

    if constexpr (!G::kSplitKeys) {
        // ---- every wave holds all keys of its rows: normalise and write its columns
        if (!loader && qrow < p.R) {
        const float poison = seq_ok ? 0.0f : __builtin_nanf("");
        const float inv = l_run == 0.0f ? 0.0f : out_scale / l_run;   // a NaN sum must propagate
        const int h = g * p.G + (qrow - qi * p.G);
        const int64_t obase = (((int64_t)b * p.n_q + qi) * p.H + h) * D + cs * DC + dcol0 + q4 * 4;
        const int64_t prow = (((int64_t)b * p.Hkv + g) * p.S + s) * p.R + qrow;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const f32x4_t v = o[db] * inv + poison;
            if (p.S == 1) {
                if constexpr (OUT_F32) {
                    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.out) + obase + db * 16) = v;
                } else {
                    uint2 wq;
                    wq.x = pack_bf16x2(v[0], v[1]);
                    wq.y = pack_bf16x2(v[2], v[3]);
                    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + obase + db * 16) = wq;
                }
            } else {
                store_partial4(p, p.ws_o + prow * D + cs * DC + dcol0 + db * 16 + q4 * 4, v);
            }
        }
        // every column split writes the row's log2-sum-exp (the same bits: all compute the
        // same scores), so each merge group finds it among its own group's writes
        if (p.S > 1 && dh == 0 && q4 == 0)
            store_partial1(p, p.ws_lse + prow, (l_run == 0.0f ? -INFINITY : m_run + log2f(l_run)) + poison);
        }
    } else {

    // ---- merge the two key halves of each row block, then write ---------------------
    // Wave (rb, kh, dh) keeps columns dcol0 + [kh*DH/2, kh*DH/2 + DH/2) and hands the
    // other half of its O^T, with its (max, sum), to its partner (rb, 1 - kh, dh).
    // The exchanged rows are DH/2 floats long: their 16-byte chunks are XOR-swizzled by
    // row so that the 16 rows of a wave's access fall on distinct LDS banks (unswizzled,
    // a row stride of 512 bytes puts all 16 on the same banks: the exchange of the
    // batched E4M3 workload took 3 us of an 18.5 us workgroup).
    constexpr int kXch = DH / 8;                                // 16-byte chunks per exchanged row
    const int xsw = l16 & (kXch >= 16 ? 15 : kXch - 1);
    __syncthreads();   // every wave is done with the stages
    float* xo = reinterpret_cast<float*>(&kst[0][0]);          // [rb][writer kh][dh][16 rows][DH/2]
    if (!loader) {
        float* dst = xo + (((rb * 2 + kh) * G::kND + dh) * 16 + l16) * (DH / 2);
#pragma unroll
        for (int db = 0; db < DB / 2; ++db) {
            const int ch = (db * 4 + q4) ^ xsw;                // columns db*16 + 4*q4 .. +3 of the half
            *reinterpret_cast<f32x4_t*>(dst + ch * 4) = pick(kh, o[db], o[DB / 2 + db]);
        }
        if (dh == 0 && q4 == 0) {
            xstat[rb][kh][0][l16] = m_run;
            xstat[rb][kh][1][l16] = l_run;
        }
    }
    __syncthreads();
    const float m_o = xstat[rb][1 - kh][0][l16];
    const float l_o = xstat[rb][1 - kh][1][l16];
    const float m_all = fmaxf(m_run, m_o);
    const float mref = m_all == -INFINITY ? 0.0f : m_all;
    const float w_me = exp2f(m_run - mref), w_o = exp2f(m_o - mref);
    // the same rounding in both waves of the pair: key half 0's term goes first
    const float l_all = kh ? __builtin_fmaf(l_o, w_o, l_run * w_me) : __builtin_fmaf(l_run, w_me, l_o * w_o);
    const float* src = xo + (((rb * 2 + (1 - kh)) * G::kND + dh) * 16 + l16) * (DH / 2);
    const int mcol = dcol0 + kh * (DH / 2);                    // the columns this wave writes

    if (!loader && qrow < p.R) {
    const float poison = seq_ok ? 0.0f : __builtin_nanf("");
    const float inv = l_all == 0.0f ? 0.0f : out_scale / l_all;   // a NaN sum must propagate
    const int h = g * p.G + (qrow - qi * p.G);
    const int64_t obase = (((int64_t)b * p.n_q + qi) * p.H + h) * D + cs * DC + mcol + q4 * 4;
    const int64_t prow = (((int64_t)b * p.Hkv + g) * p.S + s) * p.R + qrow;
#pragma unroll
    for (int db = 0; db < DB / 2; ++db) {
        const f32x4_t other = *reinterpret_cast<const f32x4_t*>(src + ((db * 4 + q4) ^ xsw) * 4);
        const f32x4_t mine = pick(kh, o[DB / 2 + db], o[db]);
        // key half 0's term first whichever wave finalises the column, so that the
        // result does not depend on how a launch splits the columns
        const f32x4_t h0 = pick(kh, other, mine), h1 = pick(kh, mine, other);
        const float w0 = kh ? w_o : w_me, w1 = kh ? w_me : w_o;
        f32x4_t num;
#pragma unroll
        for (int e = 0; e < 4; ++e) num[e] = __builtin_fmaf(h0[e], w0, h1[e] * w1);
        const f32x4_t v = num * inv + poison;
        if (p.S == 1) {
            if constexpr (OUT_F32) {
                *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.out) + obase + db * 16) = v;
            } else {
                uint2 wq;
                wq.x = pack_bf16x2(v[0], v[1]);
                wq.y = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + obase + db * 16) = wq;
            }
        } else {
            store_partial4(p, p.ws_o + prow * D + cs * DC + mcol + db * 16 + q4 * 4, v);
        }
    }
    // every column split writes the row's log2-sum-exp (the same bits: all compute the
    // same scores), so each merge group finds it among its own group's writes
    if (p.S > 1 && kh == 0 && dh == 0 && q4 == 0)
        store_partial1(p, p.ws_lse + prow, (l_all == 0.0f ? -INFINITY : m_all + log2f(l_all)) + poison);
    }
    }

    // ---- fused append: one workgroup per (problem, KV head) copies the n_q new K and V
    //      rows into the cache (no workgroup of this launch reads those cache rows: the
    //      keys at the new positions come from k_new / v_new).  Sequences and blocks
    //      outside the valid range are not written, as by the append call.
    if (!FP8 && p.k_new != nullptr && rc == 0 && cs == 0 && s == 0 && seq_ok) {
        const int per = p.n_q * G::kCpr;                  // 16-byte pieces of one tensor's rows
        for (int idx = tid; idx < 2 * per; idx += NT) {
            const bool is_v = idx >= per;
            const int r = is_v ? idx - per : idx;
            const int i = r / G::kCpr, c = r - i * G::kCpr;
            const int j = pos0 + i;
            const int blk = p.bs_log2 >= 0 ? j >> p.bs_log2 : j / p.bs;
            const int off = j - blk * p.bs;
            const int phys = p.block_table[(int64_t)b * p.max_blocks + blk];
            if (phys < 0 || phys >= p.num_blocks) continue;
            const int64_t src = (((int64_t)b * p.n_q + i) * p.Hkv + g) * G::kRowB + c * 16;
            const int64_t dst = ((int64_t)(phys * p.Hkv + g) * p.bs + off) * G::kRowB + c * 16;
            const uint4 w = *reinterpret_cast<const uint4*>(
                reinterpret_cast<const unsigned char*>(is_v ? p.v_new : p.k_new) + src);
            *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(is_v ? p.v_dst : p.k_dst) + dst) = w;
        }
    }

    // ---- split launches: the last workgroup of the (row chunk, column split) group
    //      combines the group's partials
    if (p.counters != nullptr) merge_if_last<D, OUT_F32, NT>(p, b, g, rc, cs);
}



template <int D, int KT, bool WITH_FP8, int RB, int CS = 1>
int launch_dk(const PartitionParams& p, int grid, hipStream_t st) {
    const bool fp8 = p.kv_dtype == SWATTN_FP8_E4M3;
    const bool of32 = p.out_dtype == SWATTN_F32;
    const dim3 grd((unsigned)(p.B * p.Hkv), (unsigned)(p.row_chunks * CS), (unsigned)p.S);
    if ((int64_t)grd.x * grd.y * grd.z != grid) return (int)hipErrorInvalidValue;
    if constexpr (WITH_FP8) {
        if (fp8) {
            const dim3 blk(Geo<D, true, KT, RB, CS>::kNT);
            if (of32)
                hipLaunchKernelGGL((partition_mfma_kernel<D, true, true, KT, RB, CS>), grd, blk, 0, st, p);
            else
                hipLaunchKernelGGL((partition_mfma_kernel<D, true, false, KT, RB, CS>), grd, blk, 0, st, p);
            return (int)hipGetLastError();
        }
    }
    if (fp8) return (int)hipErrorInvalidValue;
    const dim3 blk(Geo<D, false, KT, RB, CS>::kNT);
    if (of32)
        hipLaunchKernelGGL((partition_mfma_kernel<D, false, true, KT, RB, CS>), grd, blk, 0, st, p);
    else
        hipLaunchKernelGGL((partition_mfma_kernel<D, false, false, KT, RB, CS>), grd, blk, 0, st, p);
    return (int)hipGetLastError();
}

template <int D>
int launch_d(const PartitionParams& p, int grid, hipStream_t st) {
    // 32-key tiles exist for the one case where a 64-key workgroup fills a CU's LDS:
    // bfloat16 caches with head_dim 256
    if constexpr (D == 256) {
        if (p.tile_keys == 32 && p.kv_dtype == SWATTN_BF16 && p.rows_per_chunk == 32 && p.col_splits == 1)
            return launch_dk<D, 32, false, 2>(p, grid, st);
        // 64-row chunks (bfloat16 caches): 64-key tiles at one workgroup per CU while the
        // grid fits the CUs, else 32-key tiles at two per CU
        if (p.rows_per_chunk == 64) {
            if (p.kv_dtype != SWATTN_BF16 || p.col_splits != 1) return (int)hipErrorInvalidValue;
            return p.tile_keys == 64 ? launch_dk<D, 64, false, 4>(p, grid, st)
                                     : launch_dk<D, 32, false, 4>(p, grid, st);
        }
        if (p.tile_keys != 64) return (int)hipErrorInvalidValue;
        // 16-row chunks, and 32-row chunks split by columns: bfloat16 and E4M3 caches
        if (p.rows_per_chunk == 16)
            return p.col_splits == 4   ? launch_dk<D, 64, true, 1, 4>(p, grid, st)
                   : p.col_splits == 2 ? launch_dk<D, 64, true, 1, 2>(p, grid, st)
                                       : launch_dk<D, 64, true, 1, 1>(p, grid, st);
        if (p.rows_per_chunk == 32)
            return p.col_splits == 4   ? launch_dk<D, 64, true, 2, 4>(p, grid, st)
                   : p.col_splits == 2 ? launch_dk<D, 64, true, 2, 2>(p, grid, st)
                                       : launch_dk<D, 64, true, 2, 1>(p, grid, st);
        return (int)hipErrorInvalidValue;
    }
    if (p.tile_keys == 64 && p.rows_per_chunk == 32 && p.col_splits == 1) return launch_dk<D, 64, true, 2>(p, grid, st);
    return (int)hipErrorInvalidValue;
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
