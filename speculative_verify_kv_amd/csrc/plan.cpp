// swattn_plan / swattn_workspace_bytes: argument validation and launch planning.
// Pure host code: no HIP runtime call, no allocation.

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "swattn.h"
#include "swattn_internal.h"

namespace swattn {

namespace {

constexpr int64_t kFillTarget = 512;   // partition workgroups wanted in flight (2 per CU)
constexpr int64_t kMfmaFewUnits = 16;  // matrix-core launches this small split every tile off
constexpr bool kMfmaHalfRows = true;    // 16-row chunks for launches that leave CUs idle
// Matrix cores also below 16 rows (plain decode): the 16-row tile is mostly padding,
// but the call is bound by its chain of key loads, which that kernel issues a whole
// tile at a time (24-layer decode, n_q 1: 27.5 -> 11.0 us; one layer: 27 -> 8.9 us).
constexpr bool kMfmaSmallRows = true;
// 64-row chunks (32-key tiles) for bfloat16 caches of head_dim 256 with at least 64
// query rows per KV head: every K/V tile then serves twice the rows of a 32-row chunk.
constexpr bool kMfmaTallRows = true;
constexpr int64_t kFusedMaxPartialBytes = 16 * 1024;   // automatic fused merge up to this much per chunk

bool dtype_in(int v, std::initializer_list<int> ok) {
    for (int o : ok)
        if (v == o) return true;
    return false;
}

// v limited to [lo, hi]; where the bounds cross, the lower one wins (split counts: the
// least that keeps every split within its workgroup's key table beats any preference)
int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return std::max(lo, std::min(v, hi)); }

}  // namespace

swattn_status_t validate_desc(const swattn_desc_t* d, int32_t n_q, int32_t window, int32_t max_nq) {
    if (!d) return SWATTN_ERR_NULL;
    if (d->batch < 1 || d->num_heads < 1 || d->num_kv_heads < 1 ||
        d->num_heads % d->num_kv_heads != 0)
        return SWATTN_ERR_SHAPE;
    if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return SWATTN_ERR_SHAPE;
    if (d->block_size < 1 || d->max_blocks_per_seq < 1 || d->num_blocks < 1 || d->max_ctx_len < 1)
        return SWATTN_ERR_SHAPE;
    if ((int64_t)d->max_ctx_len > (int64_t)d->max_blocks_per_seq * d->block_size)
        return SWATTN_ERR_SHAPE;
    // cache rows are indexed with 32-bit integers inside the kernels
    if ((int64_t)d->num_blocks * d->num_kv_heads * d->block_size > INT32_MAX) return SWATTN_ERR_SHAPE;
    if ((int64_t)d->max_blocks_per_seq * d->block_size > INT32_MAX) return SWATTN_ERR_SHAPE;
    if (n_q < 1 || n_q > max_nq) return SWATTN_ERR_NQ;
    if (window < 1) return SWATTN_ERR_WINDOW;
    if (d->max_ctx_len < n_q) return SWATTN_ERR_CTX;
    if (!dtype_in(d->q_dtype, {SWATTN_F32, SWATTN_BF16})) return SWATTN_ERR_DTYPE;
    if (!dtype_in(d->kv_dtype, {SWATTN_F32, SWATTN_BF16, SWATTN_FP8_E4M3})) return SWATTN_ERR_DTYPE;
    if (!dtype_in(d->out_dtype, {SWATTN_F32, SWATTN_BF16})) return SWATTN_ERR_DTYPE;
    const bool fp8 = d->kv_dtype == SWATTN_FP8_E4M3;
    if (fp8 && (!d->k_scale || !d->v_scale)) return SWATTN_ERR_DTYPE;
    if (!fp8 && (d->k_scale || d->v_scale)) return SWATTN_ERR_DTYPE;
    if (d->num_splits < 0) return SWATTN_ERR_ARG;
    if (!dtype_in(d->variant, {SWATTN_VARIANT_AUTO, SWATTN_VARIANT_VALU, SWATTN_VARIANT_MFMA}))
        return SWATTN_ERR_ARG;
    if (!dtype_in(d->merge, {SWATTN_MERGE_AUTO, SWATTN_MERGE_KERNEL, SWATTN_MERGE_FUSED})) return SWATTN_ERR_ARG;
    if (d->variant == SWATTN_VARIANT_MFMA &&
        (d->q_dtype != SWATTN_BF16 || d->kv_dtype == SWATTN_F32))
        return SWATTN_ERR_DTYPE;
    return SWATTN_OK;
}

swattn_status_t make_plan(const swattn_desc_t* d, int32_t n_q, int32_t window, int32_t max_nq,
                          swattn_plan_t* out) {
    swattn_status_t st = validate_desc(d, n_q, window, max_nq);
    if (st != SWATTN_OK) return st;
    if (!out) return SWATTN_ERR_NULL;

    const int64_t G = d->num_heads / d->num_kv_heads;
    const int64_t R = (int64_t)n_q * G;                       // query rows per (problem, KV head)
    const int64_t D = d->head_dim;
    const bool mfma_ok = d->q_dtype == SWATTN_BF16 && d->kv_dtype != SWATTN_F32;

    int variant = d->variant;
    if (variant == SWATTN_VARIANT_AUTO)
        variant = (mfma_ok && (kMfmaSmallRows || R >= 16)) ? SWATTN_VARIANT_MFMA : SWATTN_VARIANT_VALU;

    // A row chunk scans the union of its own rows' windows: its queries (at most
    // (rows_per_chunk - 1) / G + 2 of them, fewer when n_q is smaller) add one key each
    // to the window.
    const int64_t rpc = variant == SWATTN_VARIANT_MFMA ? kMfmaRows : kValuRowsPerChunk;
    const int64_t qpc = std::min<int64_t>(n_q, (rpc - 1) / G + 2);
    const int64_t U = std::min<int64_t>(d->max_ctx_len, (int64_t)window + qpc - 1);   // keys per chunk

    int64_t rows_per_chunk, S;
    int64_t col_splits = 1;
    int64_t tile_keys = 0;
    const bool forced_geo = d->rows_per_chunk != 0 || d->col_splits != 0;
    if (forced_geo) {
        if (variant != SWATTN_VARIANT_MFMA) return SWATTN_ERR_ARG;
        if (!dtype_in(d->rows_per_chunk, {0, 16, 32, 64}) || !dtype_in(d->col_splits, {0, 1, 2, 4})) return SWATTN_ERR_ARG;
        if ((d->rows_per_chunk == 16 || d->rows_per_chunk == 64 || d->col_splits > 1) && d->head_dim != 256)
            return SWATTN_ERR_ARG;
        // 64-row chunks: bfloat16 caches, one workgroup per chunk
        if (d->rows_per_chunk == 64 && (d->kv_dtype != SWATTN_BF16 || d->col_splits > 1)) return SWATTN_ERR_ARG;
    }
    if (variant == SWATTN_VARIANT_MFMA) {
        rows_per_chunk = kMfmaRows;
        const int64_t s_min = (U + kMfmaMaxKeys - 1) / kMfmaMaxKeys;
        const int64_t chunks = (R + kMfmaRows - 1) / kMfmaRows;
        const int64_t units = (int64_t)d->batch * d->num_kv_heads * chunks;
        if (d->num_splits > 0)
            S = clamp64(d->num_splits, s_min, std::max<int64_t>(s_min, (U + 15) / 16));
        else if (units <= kMfmaFewUnits) {
            // A launch this small leaves most CUs idle and its time is one workgroup's
            // chain of tiles: one tile (64 keys) per split shortens the chain more than
            // the merge costs when the partials are small enough for the fused merge
            // (one layer of plain decode: 9.5 -> 7.3 us).  Behind a merge kernel the
            // split costs more than it saves (the 24-layer step of per-layer verify
            // calls: 298 us at S = 4, 289 us at S = 1).
            // Keys are counted over the union of the chunk that will run (16 rows where
            // they fit), and the partials per merge group, whose columns the chunk's
            // column splits share (one layer of the verify step: 16-row chunks split four
            // ways by columns, S = 3, 4 KiB per group: 8.45 -> 7.97 us).
            const bool half16 = kMfmaHalfRows && d->head_dim == 256;
            const int64_t qpc16 = std::min<int64_t>(n_q, (kMfmaRows / 2 - 1) / G + 2);
            const int64_t U_c = half16 ? std::min<int64_t>(d->max_ctx_len, (int64_t)window + qpc16 - 1) : U;
            S = clamp64((U_c + 63) / 64, s_min, 8);
            const int64_t g16s = (int64_t)d->batch * d->num_kv_heads * ((R + 15) / 16) * S;
            const bool half = half16 && g16s <= kComputeUnits;
            const int64_t cs_c = !half ? 1 : (4 * g16s <= kComputeUnits ? 4 : (2 * g16s <= kComputeUnits ? 2 : 1));
            const int64_t chunk_rows = std::min<int64_t>(R, half ? kMfmaRows / 2 : kMfmaRows);
            if (chunk_rows * (D / cs_c) * S * 4 > kFusedMaxPartialBytes) S = s_min;
        }
        else
            // While the launch leaves CUs idle, split long key ranges further, down to
            // 256 keys (four tiles) per split: a shorter chain per workgroup for the
            // cost of a merge (full context 1024: 30.7 -> 25.5 us at S = 4).
            S = std::max(s_min, std::min(kComputeUnits / units, (U + 255) / 256));
        // Head_dim 256 launches whose 16-row chunks fit the CUs take them: two workgroups
        // share a 32-row chunk's keys, each with half the matrix work.  Where they fit
        // twice or four times over, each 16-row chunk is also split over two or four
        // workgroups by output columns (each reading all K rows and its part of every V
        // row).  The outputs stay disjoint, so nothing merges (one verify step of 24
        // layers: 32-row chunks 15.0 us, 16-row chunks 12.1 us, split by columns too
        // 11.2 us; plain decode 12.1 -> 10.4 us).  Otherwise bfloat16 launches with 64
        // rows or more per KV head take 64-row chunks, whose K/V tiles serve twice the
        // rows (prefill of 512 positions 99.6 -> 68.6 us, wide verify 20.3 -> 18.3 us).
        const int64_t g16 = (int64_t)d->batch * d->num_kv_heads * ((R + 15) / 16) * S;
        if (kMfmaHalfRows && d->head_dim == 256 && g16 <= kComputeUnits) {
            rows_per_chunk = kMfmaRows / 2;
            col_splits = 4 * g16 <= kComputeUnits ? 4 : (2 * g16 <= kComputeUnits ? 2 : 1);
        } else if (kMfmaTallRows && d->head_dim == 256 && d->kv_dtype == SWATTN_BF16 && R >= 2 * kMfmaRows) {
            rows_per_chunk = 2 * kMfmaRows;
        }
        if (d->rows_per_chunk != 0) rows_per_chunk = d->rows_per_chunk;
        if (d->col_splits != 0) col_splits = d->col_splits;
        if (rows_per_chunk == 64) col_splits = 1;
        // A taller chunk scans a longer union of windows: keep each split within the
        // workgroup's cache-row table.
        if (rows_per_chunk > kMfmaRows) {
            const int64_t qpc_t = std::min<int64_t>(n_q, (rows_per_chunk - 1) / G + 2);
            const int64_t U_t = std::min<int64_t>(d->max_ctx_len, (int64_t)window + qpc_t - 1);
            S = std::max(S, (U_t + kMfmaMaxKeys - 1) / kMfmaMaxKeys);
        }
        // Tiles of 64 keys, or 32 where a 64-key workgroup needs a CU's whole LDS (bfloat16
        // cache, head_dim 256, 32-row chunks, no column split) and there are more
        // workgroups than CUs: 32-key tiles let two workgroups share a CU.
        const bool one_per_cu = d->kv_dtype == SWATTN_BF16 && d->head_dim == 256;
        const int64_t wgs = (int64_t)d->batch * d->num_kv_heads * ((R + rows_per_chunk - 1) / rows_per_chunk) * S;
        // 64-row chunks: 64-key tiles (eight waves, one workgroup per CU) while the grid
        // fits the CUs, else 32-key tiles (four waves, two workgroups per CU)
        tile_keys = (one_per_cu && rows_per_chunk >= kMfmaRows && col_splits == 1 && wgs > kComputeUnits) ? 32 : 64;
    } else {
        rows_per_chunk = kValuRowsPerChunk;
        const int64_t row_chunks = (R + rows_per_chunk - 1) / rows_per_chunk;
        const int64_t units = (int64_t)d->batch * d->num_kv_heads * row_chunks;
        const int64_t s_min = (U + kValuMaxKeys - 1) / kValuMaxKeys;
        const int64_t s_cap = std::max<int64_t>(s_min, (U + kValuKeyRound - 1) / kValuKeyRound);
        if (d->num_splits > 0)
            S = clamp64(d->num_splits, s_min, U);
        else
            S = clamp64((kFillTarget + units - 1) / units, s_min, s_cap);
    }
    // Every split of every row chunk within its workgroup's key table (the rules above
    // guarantee it; a plan that broke it would overrun the table in LDS)
    {
        const int64_t qpc_f = std::min<int64_t>(n_q, (rows_per_chunk - 1) / G + 2);
        const int64_t U_f = std::min<int64_t>(d->max_ctx_len, (int64_t)window + qpc_f - 1);
        const int64_t table = variant == SWATTN_VARIANT_MFMA ? kMfmaMaxKeys : kValuMaxKeys;
        if ((U_f + S - 1) / S > table) return SWATTN_ERR_SHAPE;
    }
    const int64_t row_chunks = (R + rows_per_chunk - 1) / rows_per_chunk;
    const int64_t grid = (int64_t)d->batch * d->num_kv_heads * row_chunks * col_splits * S;
    if (grid > INT32_MAX) return SWATTN_ERR_SHAPE;
    // the matrix-core kernel launches a (B * Hkv, row chunks, splits) grid
    if (variant == SWATTN_VARIANT_MFMA && (row_chunks * col_splits > 65535 || S > 65535)) return SWATTN_ERR_SHAPE;

    const int64_t rows_total = (int64_t)d->batch * d->num_kv_heads * R;
    const int64_t merge_rows_per_wg = (kMergeThreads * 4) / D;   // D/4 threads per row
    int64_t merge_grid = 0;
    int32_t fused = 0;
    size_t ws = 0;
    if (S > 1) {
        // The last workgroup of each merge group (row chunk x column split) combines the
        // group's partials (no second launch) when the groups fit the counter region and
        // a group's partials are small (at most kFusedMaxPartialBytes: one workgroup
        // reads them all, from past its L2); otherwise a merge kernel spreads the
        // combination over many workgroups.  Measured (MI355X, cold): tiny decode at
        // S = 3 (1.5 KiB of partials), 13.5 -> 12.6 us; one layer of the verify step at
        // S = 4 (128 KiB), +2 us per call; full context 4096 at S = 8 (256 KiB), 49 -> 54 us.
        const int64_t groups_total = (int64_t)d->batch * d->num_kv_heads * row_chunks * col_splits;
        if (d->merge == SWATTN_MERGE_FUSED && groups_total > kMergeCounters) return SWATTN_ERR_SHAPE;
        const int64_t group_partial_bytes = std::min<int64_t>(rows_per_chunk, R) * (D / col_splits) * S * 4;
        fused = d->merge == SWATTN_MERGE_FUSED ||
                (d->merge == SWATTN_MERGE_AUTO && groups_total <= kMergeCounters &&
                 group_partial_bytes <= kFusedMaxPartialBytes);
        if (!fused) {
            merge_grid = (rows_total + merge_rows_per_wg - 1) / merge_rows_per_wg;
            if (merge_grid > INT32_MAX) return SWATTN_ERR_SHAPE;
        }
        // layout: [arrival counters][partial outputs][partial log2-sum-exps]
        const int64_t o_bytes = ((rows_total * S * D * 4) + 255) / 256 * 256;
        ws = (size_t)(SWATTN_WORKSPACE_COUNTER_BYTES + o_bytes + rows_total * S * 4);
    }
    out->variant = variant;
    out->num_splits = (int32_t)S;
    out->rows_per_chunk = (int32_t)rows_per_chunk;
    out->row_chunks = (int32_t)row_chunks;
    out->grid = (int32_t)grid;
    out->merge_grid = (int32_t)merge_grid;
    out->fused_merge = fused;
    out->workspace_bytes = ws;
    out->col_splits = (int32_t)col_splits;
    out->tile_keys = (int32_t)tile_keys;
    return SWATTN_OK;
}

}  // namespace swattn

extern "C" {

swattn_status_t swattn_plan(const swattn_desc_t* desc, int32_t n_q, int32_t window, swattn_plan_t* plan) {
    if (!plan) return SWATTN_ERR_NULL;
    swattn_plan_t tmp;
    swattn_status_t st = swattn::make_plan(desc, n_q, window, SWATTN_MAX_NQ, &tmp);
    if (st == SWATTN_OK) *plan = tmp;
    return st;
}

swattn_status_t swattn_prefill_plan(const swattn_desc_t* desc, int32_t n_q, int32_t window, swattn_plan_t* plan) {
    if (!plan) return SWATTN_ERR_NULL;
    swattn_plan_t tmp;
    swattn_status_t st = swattn::make_plan(desc, n_q, window, SWATTN_MAX_PREFILL_NQ, &tmp);
    if (st == SWATTN_OK) *plan = tmp;
    return st;
}

swattn_status_t swattn_workspace_bytes(const swattn_desc_t* desc, int32_t n_q, int32_t window, size_t* bytes) {
    if (!bytes) return SWATTN_ERR_NULL;
    swattn_plan_t tmp;
    swattn_status_t st = swattn::make_plan(desc, n_q, window, SWATTN_MAX_NQ, &tmp);
    if (st == SWATTN_OK) *bytes = tmp.workspace_bytes;
    return st;
}

const char* swattn_status_str(swattn_status_t s) {
    switch (s) {
        case SWATTN_OK: return "ok";
        case SWATTN_ERR_NULL: return "a required pointer is NULL";
        case SWATTN_ERR_SHAPE: return "invalid shape (batch, heads, head_dim, block sizes or max_ctx_len)";
        case SWATTN_ERR_NQ: return "n_q outside [1, 64] (verify) or [1, 512] (prefill)";
        case SWATTN_ERR_WINDOW: return "window < 1";
        case SWATTN_ERR_DTYPE: return "unsupported dtype combination (or e4m3 KV without scales, or scales without e4m3)";
        case SWATTN_ERR_ALIGN: return "a data pointer is not 16-byte aligned";
        case SWATTN_ERR_WORKSPACE: return "workspace missing or smaller than the plan needs";
        case SWATTN_ERR_CTX: return "ctx_len outside [n_q, min(max_ctx_len, max_blocks_per_seq*block_size)]";
        case SWATTN_ERR_BLOCK: return "a block id read by some window lies outside [0, num_blocks)";
        case SWATTN_ERR_HIP: return "HIP runtime error";
        case SWATTN_ERR_ARG: return "invalid argument";
        case SWATTN_ERR_SCRATCH:
            return "the plan needs more workspace than the library's static scratch (SWATTN_STATIC_SCRATCH_BYTES) holds";
    }
    return "unknown status";
}

int32_t swattn_abi_version(void) { return SWATTN_ABI_VERSION; }

}  // extern "C"
