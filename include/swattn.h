/*
 * swattn.h — C ABI of the sliding-window verify-attention library (MI355X / gfx950).
 *
 * The operation.  One call scores the n_q newest positions of B independent
 * attention problems ("sequences"; a model's layers stacked along B count as
 * separate problems) against a paged KV cache:
 *
 *   for b < B, i < n_q, h < H:
 *     p   = ctx_len[b] - n_q            (position of the first new token)
 *     t   = p + i                       (position of query i)
 *     g   = h / (H / Hkv)               (grouped-query head mapping)
 *     out[b][i][h] = sum_{t-window < j <= t} softmax_j(scale * q[b][i][h] . k_j) v_j
 *     where k_j, v_j are row (j % block_size) of KV head g in physical block
 *     block_table[b][j / block_size].
 *
 * Source: "The Fast Gemma Challenge: our verified-SOTA recipe, in full" (dev.to,
 * VIDRAFT), full manifest.json — SLIDING_WINDOW=188 and FA_SLIDING=1 (attention
 * over the most recent W tokens), SPECULATIVE_CONFIG with 7 MTP draft tokens (a
 * verify step scores the target plus 7 drafts, each causal on the ones before
 * it), SPLITKV_VERIFY / SPLITKV_VERIFY_MAX_Q=64 (the split-KV verify kernel takes
 * at most 64 queries) and MAX_MODEL_LEN=4096; and its section "What each piece
 * does, and why" (the window exists because decode is bound by KV-cache
 * bandwidth; ONEGRAPH removes launch overhead, so calls must be capturable into
 * a HIP graph).  Plain decode is n_q = 1.  The pages do not state whether the
 * current token is inside the window; it is read here as included, so window = 1
 * returns the query's own V row and window >= ctx_len is full causal attention.
 *
 * Threading and streams.  Every function is reentrant; the library keeps no
 * state between calls.  swattn_verify enqueues at most two kernels on the given
 * HIP stream and returns without synchronising or allocating, so it may be
 * captured into a HIP graph.
 */
#ifndef SWATTN_H
#define SWATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWATTN_ABI_VERSION 3
#define SWATTN_MAX_NQ 64          /* SPLITKV_VERIFY_MAX_Q of the manifest */
#define SWATTN_MAX_PREFILL_NQ 512 /* MAX_NUM_BATCHED_TOKENS of the manifest */

typedef enum {
    SWATTN_F32 = 0,               /* IEEE binary32 */
    SWATTN_BF16 = 1,              /* bfloat16 (upper half of binary32) */
    SWATTN_FP8_E4M3 = 2           /* OCP FP8 E4M3 ("e4m3fn"): bias 7, max 448, no inf */
} swattn_dtype_t;

typedef enum {
    SWATTN_OK = 0,
    SWATTN_ERR_NULL = -1,         /* a required pointer is NULL */
    SWATTN_ERR_SHAPE = -2,        /* batch/heads/head_dim/block sizes invalid, or the launch would need
                                     more than INT32_MAX workgroups (65535 splits or row chunks for the
                                     matrix-core variant) */
    SWATTN_ERR_NQ = -3,           /* n_q outside [1, SWATTN_MAX_NQ] (prefill: [1, SWATTN_MAX_PREFILL_NQ]) */
    SWATTN_ERR_WINDOW = -4,       /* window < 1 */
    SWATTN_ERR_DTYPE = -5,        /* unsupported dtype combination, or e4m3 without scales */
    SWATTN_ERR_ALIGN = -6,        /* a data pointer is not 16-byte aligned */
    SWATTN_ERR_WORKSPACE = -7,    /* workspace NULL or smaller than the plan needs */
    SWATTN_ERR_CTX = -8,          /* a ctx_len outside [n_q, min(max_ctx_len, max_blocks*block_size)] */
    SWATTN_ERR_BLOCK = -9,        /* a referenced block id outside [0, num_blocks) */
    SWATTN_ERR_HIP = -10,         /* a HIP runtime call failed */
    SWATTN_ERR_ARG = -11,         /* other invalid argument (scale not finite, bad override) */
    SWATTN_ERR_SCRATCH = -12      /* swattn_verify_noalloc: the plan's workspace exceeds
                                     SWATTN_STATIC_SCRATCH_BYTES */
} swattn_status_t;

typedef enum {
    SWATTN_VARIANT_AUTO = 0,      /* matrix cores for bf16 q with bf16/e4m3 kv, else vector ALU */
    SWATTN_VARIANT_VALU = 1,      /* fp32 vector-ALU partition kernel (any dtype) */
    SWATTN_VARIANT_MFMA = 2       /* bf16 matrix-core partition kernel (bf16 q, bf16/e4m3 kv) */
} swattn_variant_t;

/* How the partials of a split launch (S > 1) are combined. */
typedef enum {
    SWATTN_MERGE_AUTO = 0,        /* fused when a row chunk's partials are small (<= 16 KiB,
                                     e.g. decode) and the launch has few enough row chunks,
                                     else the merge kernel */
    SWATTN_MERGE_KERNEL = 1,      /* a separate merge kernel after the partition kernel */
    SWATTN_MERGE_FUSED = 2        /* the last partition workgroup of each merge group (row chunk x
                                     column split) combines; SWATTN_ERR_SHAPE when the launch has
                                     more groups (B * Hkv * row_chunks * col_splits) than
                                     counters (SWATTN_WORKSPACE_COUNTER_BYTES / 4) */
} swattn_merge_t;

/* Problem description.  Plain data; the caller owns it. */
typedef struct {
    int32_t batch;                /* B >= 1 independent problems */
    int32_t num_heads;            /* H >= 1, a multiple of num_kv_heads */
    int32_t num_kv_heads;         /* Hkv >= 1 */
    int32_t head_dim;             /* D in {64, 128, 256} */
    int32_t block_size;           /* KV positions per cache block, >= 1 */
    int32_t max_blocks_per_seq;   /* row length of block_table, >= 1 */
    int32_t num_blocks;           /* physical blocks in the KV pool, >= 1 */
    int32_t max_ctx_len;          /* host-side upper bound of ctx_len[]; used to plan splits */
    swattn_dtype_t q_dtype;       /* F32 or BF16 */
    swattn_dtype_t kv_dtype;      /* F32, BF16 or FP8_E4M3 */
    swattn_dtype_t out_dtype;     /* F32 or BF16 */
    const float* k_scale;         /* [Hkv] device fp32, required iff kv_dtype == FP8_E4M3, else NULL */
    const float* v_scale;         /* [Hkv] device fp32, same rule; stored value * scale = real value */
    int32_t num_splits;           /* 0: library chooses; > 0 forces the KV split count */
    int32_t variant;              /* swattn_variant_t; AUTO lets the library choose */
    int32_t merge;                /* swattn_merge_t: how split partials are combined */
    /* Tuning overrides of the matrix-core launch (0: library chooses).  They force a
     * geometry; SWATTN_ERR_ARG when the plan is not the matrix-core variant or the value
     * is not offered for this shape. */
    int32_t rows_per_chunk;       /* 16, 32 or 64 query rows per workgroup (16 and 64: head_dim
                                     256 only; 64: bfloat16 caches, no column split) */
    int32_t col_splits;           /* 1, 2 or 4 workgroups per row chunk, each with D/col_splits
                                     output columns (head_dim 256 only) */
} swattn_desc_t;

/* What swattn_verify will launch for a description (filled by swattn_plan). */
typedef struct {
    int32_t variant;              /* SWATTN_VARIANT_VALU or SWATTN_VARIANT_MFMA */
    int32_t num_splits;           /* S: KV splits per (problem, KV head, row chunk) */
    int32_t rows_per_chunk;       /* query rows (n_q * H/Hkv packed) per workgroup */
    int32_t row_chunks;           /* row chunks per (problem, KV head) */
    int32_t grid;                 /* workgroups of the partition kernel */
    int32_t merge_grid;           /* workgroups of the merge kernel (0 when S == 1 or fused) */
    int32_t fused_merge;          /* 1: the last partition workgroup of each merge group (row
                                     chunk x column split) to finish combines the group's S
                                     partials itself (no merge kernel) */
    size_t workspace_bytes;       /* device scratch swattn_verify needs (0 when S == 1) */
    int32_t col_splits;           /* workgroups per row chunk, each with D/col_splits output
                                     columns (matrix-core variant; 1 otherwise) */
    int32_t tile_keys;            /* keys per LDS tile of the matrix-core kernel (32 or 64;
                                     0 for the vector-ALU variant) */
} swattn_plan_t;

/* A split plan's workspace starts with this many bytes of arrival counters, the
 * same region for every plan.  They must be zero before the first call that uses
 * the workspace (swattn_workspace_init, or any zero fill); every call leaves them
 * zero, so one fill serves all later calls, with any plan. */
#define SWATTN_WORKSPACE_COUNTER_BYTES 4096

/*
 * swattn_plan — validate a description and choose the launch.  Pure host code:
 * no HIP call, no allocation; safe on a machine without a GPU.
 * Returns SWATTN_OK and fills *plan, or an error code and leaves *plan untouched.
 */
swattn_status_t swattn_plan(const swattn_desc_t* desc, int32_t n_q, int32_t window,
                            swattn_plan_t* plan);

/* Zero the arrival counters of a fresh workspace of `bytes` bytes (16-byte aligned,
 * device memory) on `stream`: one small kernel, no memset, so it may be captured in
 * a graph.  Needed once per workspace; a zero-filled allocation needs nothing. */
swattn_status_t swattn_workspace_init(void* workspace, size_t bytes, void* stream);

/* Convenience: workspace size in bytes for (desc, n_q, window); pure host code. */
swattn_status_t swattn_workspace_bytes(const swattn_desc_t* desc, int32_t n_q, int32_t window,
                                       size_t* bytes);

/*
 * swattn_verify — sliding-window attention for one verify (or decode) step.
 *
 *   q           [B][n_q][H][D]            q_dtype, device, read-only
 *   k_cache     [num_blocks][Hkv][block_size][D]  kv_dtype, device, read-only
 *   v_cache     same layout and dtype as k_cache
 *   block_table [B][max_blocks_per_seq]   int32, device; entries past a sequence's
 *                                         last block are never read
 *   ctx_len     [B] int32, device; valid positions of sequence b, counting its
 *               n_q new tokens, whose K/V must already be in the cache
 *   n_q         1 .. SWATTN_MAX_NQ (1 = decode, 1 + drafts = verify)
 *   window      >= 1 positions per query, the query's own position included
 *   scale       finite softmax scale (usually 1/sqrt(D))
 *   out         [B][n_q][H][D] out_dtype, device; fully overwritten; must not alias q
 *   workspace   device scratch of >= plan.workspace_bytes (may be NULL when that is 0);
 *               its first SWATTN_WORKSPACE_COUNTER_BYTES must be zero on entry (see
 *               swattn_workspace_init) and are zero again on completion; the rest is
 *               undefined afterwards; calls that overlap in time need separate
 *               workspaces
 *   stream      hipStream_t (NULL = default stream)
 *
 * All data pointers must be 16-byte aligned.  Host-checkable errors are returned
 * before anything is enqueued.  Device-resident preconditions are not checked on
 * this path (swattn_check_inputs does that): a sequence whose ctx_len lies
 * outside [n_q, min(max_ctx_len, max_blocks_per_seq*block_size)] gets NaN in all
 * its outputs, and a
 * window position whose block id lies outside [0, num_blocks) is read as NaN, so
 * bad inputs show in the output instead of faulting.  Launch failures return
 * SWATTN_ERR_HIP; asynchronous faults surface on the stream.
 */
swattn_status_t swattn_verify(const swattn_desc_t* desc,
                              const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* ctx_len,
                              int32_t n_q, int32_t window, float scale,
                              void* out, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * swattn_prefill_plan / swattn_prefill — the same attention for a chunk of up to
 * SWATTN_MAX_PREFILL_NQ new positions per sequence (chunked prefill).
 *
 * Source: "The Fast Gemma Challenge: our verified-SOTA recipe, in full" (dev.to,
 * VIDRAFT), full manifest.json — MAX_NUM_BATCHED_TOKENS=512 caps the tokens of one
 * engine step, prefill chunks included, while SPLITKV_VERIFY_MAX_Q=64 caps the verify
 * path; a prefill chunk therefore takes the same windowed attention with n_q above 64.
 * Arguments, layouts, ownership, alignment, workspace and error behaviour are those of
 * swattn_plan / swattn_verify, with n_q in [1, SWATTN_MAX_PREFILL_NQ].  Each 32-row
 * (or 8-row) chunk of query rows scans only the union of its own rows' windows, so the
 * work grows with n_q * window, not n_q * (window + n_q).
 */
swattn_status_t swattn_prefill_plan(const swattn_desc_t* desc, int32_t n_q, int32_t window,
                                    swattn_plan_t* plan);

swattn_status_t swattn_prefill(const swattn_desc_t* desc,
                               const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* ctx_len,
                               int32_t n_q, int32_t window, float scale,
                               void* out, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * swattn_append_kv — write the n_new new K and V rows of every sequence into the
 * paged cache, converting them to the cache's element type.
 *
 * Source: "The Fast Gemma Challenge: our verified-SOTA recipe, in full" (dev.to,
 * VIDRAFT), full manifest.json — SPECULATIVE_CONFIG (a verify step scores the target
 * token and 7 drafts, whose K/V rows must be in the cache before attention reads
 * them) and section "What each piece does, and why" (decode is bound by the KV
 * cache's bandwidth, which is why the cache may be stored in 8 bits).
 *
 *   k_new, v_new  [B][n_new][Hkv][D] new_dtype (F32 or BF16), device, read-only
 *   block_table   [B][max_blocks_per_seq] int32, device
 *   ctx_len       [B] int32, device; counts the new tokens, as in swattn_verify
 *   k_cache, v_cache  [num_blocks][Hkv][block_size][D] desc->kv_dtype, device;
 *                 only the new rows' positions are written
 *
 * Row (b, i, g) goes to position t = ctx_len[b] - n_new + i: block
 * block_table[b][t / block_size], offset t % block_size.  Conversion to the cache
 * type: bfloat16 rounds to nearest even; E4M3 stores the float32 quotient
 * value / scale[g] (correctly rounded division, desc->k_scale / v_scale) rounded to
 * the nearest E4M3 value, ties to the even code, saturating at +-448, NaN kept as
 * NaN; float32 caches store the value.  desc fields used: batch, num_kv_heads,
 * head_dim, block_size, max_blocks_per_seq, num_blocks, max_ctx_len, kv_dtype,
 * k_scale, v_scale (the others are ignored).  n_new is in [1, SWATTN_MAX_PREFILL_NQ].
 * A sequence whose ctx_len lies outside [n_new, min(max_ctx_len,
 * max_blocks_per_seq*block_size)], or a position whose block id lies outside
 * [0, num_blocks), is not written (nothing else is touched).  Host-checkable
 * errors return before anything is enqueued; the call enqueues one kernel, never
 * allocates or synchronises, and may be captured into a HIP graph.  Pointers as in
 * swattn_verify (16-byte aligned data, 4-byte aligned tables).  The new rows must
 * not overlap the cache.
 */
swattn_status_t swattn_append_kv(const swattn_desc_t* desc, const void* k_new, const void* v_new,
                                 swattn_dtype_t new_dtype, const int32_t* block_table,
                                 const int32_t* ctx_len, int32_t n_new, void* k_cache, void* v_cache,
                                 void* stream);

/*
 * swattn_append_verify — swattn_append_kv of the step's n_q new rows, then
 * swattn_verify, as one call.
 *
 * Source: "The Fast Gemma Challenge: our verified-SOTA recipe, in full" (dev.to,
 * VIDRAFT), full manifest.json — SPECULATIVE_CONFIG (the verify step's target and
 * drafts bring their own K/V rows, which their attention must already see) and
 * SPLITKV_VERIFY; section "What each piece does, and why".
 *
 * Arguments as in swattn_append_kv (k_new, v_new, new_dtype, with n_new = n_q) and
 * swattn_verify (the rest); k_cache and v_cache are written.  The result, outputs and
 * cache bytes, is that of the two calls in order.  Where the plan runs the
 * matrix-core kernel and both the new rows and the cache are bfloat16 (the append is
 * then a copy), it is one launch: keys at the new positions are read from k_new /
 * v_new, and the kernel writes those rows into the cache; otherwise the append
 * kernel runs first.  In the one-launch form the blocks holding a sequence's new
 * positions must not lie in another sequence's window (blocks are not shared with
 * a sequence that is being appended to).  Errors of either call return before
 * anything is enqueued; no allocation or synchronisation, capturable into a HIP
 * graph.
 */
swattn_status_t swattn_append_verify(const swattn_desc_t* desc, const void* q, const void* k_new, const void* v_new,
                                     swattn_dtype_t new_dtype, void* k_cache, void* v_cache,
                                     const int32_t* block_table, const int32_t* ctx_len, int32_t n_q,
                                     int32_t window, float scale, void* out, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * swattn_greedy_accept — greedy acceptance of one verify step's drafts.
 *
 * Source: "The Fast Gemma Challenge: our verified-SOTA recipe, in full" (dev.to,
 * VIDRAFT), full manifest.json — OVERRIDE_GENERATION_CONFIG (temperature 0, top_p 1,
 * top_k 0: greedy generation, so the target's token is the argmax of its logits),
 * SPECULATIVE_CONFIG (a verify step scores the last accepted token and 7 drafts) and
 * FUSED_SPARSE_ARGMAX (the argmax is fused into the step instead of sampled).
 *
 *   logits      [B][n_q][vocab] logits_dtype (F32 or BF16), device, read-only; the
 *               target's logits after each of the step's n_q inputs
 *   draft_ids   [B][n_q - 1] int32, device; draft_ids[b][j] is the drafter's guess for
 *               the token after input j (may be NULL when n_q == 1)
 *   target_ids  [B][n_q] int32, device, written: argmax_v logits[b][i][v], the lowest
 *               index among equal maxima; a NaN counts as larger than every number (the
 *               first NaN wins); -0 equals +0
 *   accepted    [B] int32, device, written: the largest a <= n_q - 1 such that
 *               draft_ids[b][j] == target_ids[b][j] for every j < a
 *   next_token  [B] int32, device, written: target_ids[b][accepted[b]]
 *   workspace   device scratch of >= swattn_greedy_accept_workspace(B, n_q, vocab) bytes,
 *               8-byte aligned; contents undefined afterwards
 *
 * n_q in [1, SWATTN_MAX_NQ], vocab >= 1.  logits aligned to its element size.  Two
 * kernels on the stream (a chunked argmax and a per-sequence finalize); no
 * allocation or synchronisation, capturable into a HIP graph.  Host-checkable errors
 * return before anything is enqueued.
 */
swattn_status_t swattn_greedy_accept_workspace(int32_t batch, int32_t n_q, int32_t vocab, size_t* bytes);

swattn_status_t swattn_greedy_accept(const void* logits, swattn_dtype_t logits_dtype, int32_t batch,
                                     int32_t n_q, int32_t vocab, const int32_t* draft_ids,
                                     int32_t* target_ids, int32_t* accepted, int32_t* next_token,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * swattn_check_inputs — debug check of the device-resident preconditions (n_q up to
 * SWATTN_MAX_PREFILL_NQ).  Copies ctx_len and block_table to the host (synchronising the stream) and
 * returns SWATTN_ERR_CTX if some ctx_len[b] lies outside
 * [n_q, min(max_ctx_len, max_blocks_per_seq*block_size)], SWATTN_ERR_BLOCK if a block id that a
 * window reads lies outside [0, num_blocks), SWATTN_OK otherwise.  Allocates
 * host memory only; not for use under graph capture.
 */
swattn_status_t swattn_check_inputs(const swattn_desc_t* desc, const int32_t* block_table,
                                    const int32_t* ctx_len, int32_t n_q, int32_t window,
                                    void* stream);

/*
 * swattn_verify_noalloc — swattn_verify without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments, layouts, semantics, results
 * and errors are those of swattn_verify (the same plan and kernels), except that a
 * split plan's workspace is a device array inside the library, one per GPU, of
 * SWATTN_STATIC_SCRATCH_BYTES bytes, held until the process ends.  The call never
 * allocates or frees (nor does anything it calls).  A plan whose workspace is larger
 * returns SWATTN_ERR_SCRATCH before anything is enqueued (swattn_plan tells the
 * size; num_splits or merge choices change it).  The first call on a device that
 * needs the array also enqueues, on `stream`, a small kernel that zeroes its arrival
 * counters; every call leaves them zero.  Calls on one GPU share its array: calls
 * that overlap in time on one GPU (other streams or threads) race and must not be
 * issued.
 */
#define SWATTN_STATIC_SCRATCH_BYTES (16u << 20)

swattn_status_t swattn_verify_noalloc(const swattn_desc_t* desc,
                                      const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* ctx_len,
                                      int32_t n_q, int32_t window, float scale,
                                      void* out, void* stream);

/*
 * swattn_window_gather — measurement aid: the data movement of swattn_verify without
 * its arithmetic.  For each (problem, KV head) it reads the K and V rows of the union
 * of the n_q queries' windows through the block table (the same 16-byte global-to-LDS
 * loads as the attention kernel, all requested at once), reads the problem's Q rows,
 * and writes zeros over its rows of `out`: exactly the bytes counted as the verify
 * call's algorithmic traffic, so its time is the data-movement floor of that paged
 * layout and launch shape.  `parts` (1..16, else SWATTN_ERR_ARG) workgroups share each
 * (problem, KV head), each taking a contiguous slice of its window rows, Q rows and
 * output rows.  Other arguments and host-side checks as swattn_verify (no workspace);
 * `out` receives zeros.  A window of more than 1024 positions is read over
 * its first 1024, and at most 512 query rows per KV head.  Source of the window rule:
 * "The Fast Gemma Challenge: our verified-SOTA recipe, in full", manifest
 * SLIDING_WINDOW, SPECULATIVE_CONFIG; "What each piece does, and why" (decode is bound
 * by the KV cache's bandwidth).
 */
swattn_status_t swattn_window_gather(const swattn_desc_t* desc,
                                     const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_table, const int32_t* ctx_len,
                                     int32_t n_q, int32_t window, int32_t parts, void* out, void* stream);

/*
 * swattn_stream_read — measurement aid: a plain contiguous read of `bytes` bytes at
 * `src` (device memory, 16-byte aligned, `bytes` a non-negative multiple of 16), the
 * time HBM alone sets for moving a call's byte count, to set beside
 * swattn_window_gather's paged floor.  `grid` (1..65536) workgroups of 1024 threads
 * stream it from the first cycle, thread t of the grid reading the 16-byte chunks
 * t, t + 1024*grid, t + 2*1024*grid, ...; workgroup w writes xor_out[4w .. 4w+3] (device
 * memory the caller owns, 4-byte aligned, 4*grid words): the xor, word by word, of the
 * 16-byte chunks it read (zeros if none), so that a caller can check the read.  With
 * xor_out NULL nothing is written (the form to time: reads only).  Returns
 * SWATTN_ERR_NULL (src NULL), SWATTN_ERR_ALIGN or SWATTN_ERR_ARG before enqueuing
 * anything when those conditions fail, SWATTN_ERR_HIP if the launch fails.  Context:
 * "What each piece does, and why" in "The Fast Gemma Challenge: our verified-SOTA
 * recipe, in full" (decode is bound by the KV cache's bandwidth).
 */
swattn_status_t swattn_stream_read(const void* src, int64_t bytes, int32_t grid, uint32_t* xor_out, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* swattn_status_str(swattn_status_t status);

/* SWATTN_ABI_VERSION of the loaded library. */
int32_t swattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SWATTN_H */
