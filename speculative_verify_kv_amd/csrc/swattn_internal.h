// Internal interface between the host library (plan / api) and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "swattn.h"

namespace swattn {

// Launch geometry shared by the planner and the kernels.
constexpr int kWaveSize = 64;
constexpr int kBlockThreads = 256;           // 4 waves: VALU partition, argmax, append and fill kernels
constexpr int kMergeThreads = 256;           // merge kernel workgroup (D/4 threads per row)
constexpr int kMfmaRows = 32;                // query rows per matrix-core workgroup (two 16-row tiles)
constexpr int kMfmaMaxKeys = 512;            // keys per matrix-core workgroup (cache-row table in LDS)
constexpr int kComputeUnits = 256;           // MI355X
constexpr int kValuRowsPerChunk = 8;         // query rows per VALU workgroup
constexpr int kValuMaxKeys = 256;            // keys per VALU workgroup (score buffer size)
constexpr int kValuKeyRound = 64;            // keys scored per round in the VALU kernel
// Split launches keep one arrival counter per (problem, KV head, row chunk) at the
// start of the workspace, in a region of fixed size for every plan, so that no plan's
// partials ever overwrite another plan's counters.  Launches with more units than
// counters use the separate merge kernel instead.
constexpr int kMergeCounters = SWATTN_WORKSPACE_COUNTER_BYTES / 4;

// Everything a partition kernel needs, passed by value.
struct PartitionParams {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* block_table;
    const int32_t* ctx_len;
    const float* k_scale;
    const float* v_scale;
    void* out;
    float* ws_o;          // [B*Hkv][S][R][D] normalised partial outputs (S > 1)
    float* ws_lse;        // [B*Hkv][S][R] log2-sum-exp of each partial (S > 1)
    int32_t* counters;    // [B*Hkv][row_chunks] arrivals (fused merge), else NULL
    // Fused append (matrix-core kernel, bfloat16 rows and cache): the n_q new rows
    // [B][n_q][Hkv][D] of every sequence, read for the keys at the new positions and
    // written into the cache through k_dst / v_dst (the same caches as k / v); NULL
    // otherwise.
    const void* k_new;
    const void* v_new;
    void* k_dst;
    void* v_dst;
    int32_t B, H, Hkv, G, D, bs, max_blocks, num_blocks;
    int32_t bs_log2;      // log2(bs) when bs is a power of two, else -1
    int32_t n_q, window, R, max_ctx;
    int32_t S, rows_per_chunk, row_chunks;
    int32_t col_splits;   // workgroups per row chunk splitting its output columns (1, 2 or 4)
    int32_t q_dtype, kv_dtype, out_dtype;
    float scale_log2;     // scale * log2(e)
    int32_t tile_keys;    // matrix-core kernel: keys per tile, 32 or 64
};

struct MergeParams {
    const float* ws_o;
    const float* ws_lse;
    void* out;
    int32_t B, H, Hkv, G, D, n_q, R, S;
    int32_t out_dtype;
};

// KV-cache append (kv_append.hip).
struct AppendParams {
    const void* k_new;    // [B][n_new][Hkv][D] new_dtype
    const void* v_new;
    void* k_cache;        // [num_blocks][Hkv][bs][D] kv_dtype
    void* v_cache;
    const int32_t* block_table;
    const int32_t* ctx_len;
    const float* k_scale;
    const float* v_scale;
    int32_t B, Hkv, D, bs, max_blocks, num_blocks, max_ctx, n_new;
    int32_t new_dtype, kv_dtype;
};

// Greedy acceptance (accept.hip).
constexpr int kAcceptChunk = 8192;           // logits per workgroup of the argmax pass
constexpr int kAcceptMaxNq = 64;             // positions per sequence (the verify cap)
struct AcceptParams {
    const void* logits;   // [B][n_q][vocab] float32 or bfloat16
    const int32_t* draft_ids;   // [B][n_q - 1]
    int32_t* target_ids;        // [B][n_q]
    int32_t* accepted;          // [B]
    int32_t* next_token;        // [B]
    uint64_t* partial;          // [B * n_q][nchunk] argmax keys (workspace)
    int32_t B, n_q, vocab, nchunk, logits_dtype, vec_ok;
};

// Geometry helpers used by both the planner and the host launch code.
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Planning and the attention call of swattn_verify / swattn_prefill (plan.cpp, api.cpp):
// checks, plan and launches on `stream`, with the given workspace.
swattn_status_t make_plan(const swattn_desc_t* d, int32_t n_q, int32_t window, int32_t max_nq,
                          swattn_plan_t* out);
swattn_status_t attend(const swattn_desc_t* d, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* ctx_len, int32_t n_q, int32_t window,
                       float scale, void* out, void* workspace, size_t workspace_bytes, void* stream,
                       int32_t max_nq);
// The same call in two halves: every check and the launch parameters (nothing is
// enqueued), then the launches.
struct AttendCall {
    swattn_plan_t plan;
    PartitionParams p;
    MergeParams m;
};
swattn_status_t prepare_attend(const swattn_desc_t* d, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* ctx_len, int32_t n_q, int32_t window,
                               float scale, void* out, void* workspace, size_t workspace_bytes, int32_t max_nq,
                               AttendCall* call);
swattn_status_t launch_attend(const AttendCall& call, void* stream);

// Kernel launchers (defined in the .hip files).  They return a hipError_t as int.
int launch_partition_mfma(const PartitionParams& p, int grid, void* stream);
int launch_partition_valu(const PartitionParams& p, int grid, void* stream);
int launch_merge(const MergeParams& p, int grid, void* stream);
int launch_zero_words(int32_t* w, int n, void* stream);
int launch_kv_append(const AppendParams& p, int grid, void* stream);
int launch_accept(const AcceptParams& p, int grid1, void* stream);

}  // namespace swattn
