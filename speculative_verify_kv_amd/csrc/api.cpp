// swattn_verify / swattn_check_inputs: host side of the C ABI.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <vector>

#include "swattn.h"
#include "swattn_internal.h"

namespace swattn {
swattn_status_t validate_desc(const swattn_desc_t* d, int32_t n_q, int32_t window, int32_t max_nq);
swattn_status_t make_plan(const swattn_desc_t* d, int32_t n_q, int32_t window, int32_t max_nq,
                          swattn_plan_t* out);

namespace {

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

int dtype_bytes(int dt) { return dt == SWATTN_F32 ? 4 : (dt == SWATTN_BF16 ? 2 : 1); }

}  // namespace
}  // namespace swattn

namespace swattn {

// An attention call, checked and laid out (verify or prefill: they differ only in the
// n_q cap); nothing is enqueued.
swattn_status_t prepare_attend(const swattn_desc_t* d, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* ctx_len, int32_t n_q, int32_t window,
                               float scale, void* out, void* workspace, size_t workspace_bytes, int32_t max_nq,
                               AttendCall* call) {
    swattn_plan_t& plan = call->plan;
    swattn_status_t st = make_plan(d, n_q, window, max_nq, &plan);
    if (st != SWATTN_OK) return st;
    if (!q || !k_cache || !v_cache || !block_table || !ctx_len || !out) return SWATTN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
        !aligned(block_table, 4) || !aligned(ctx_len, 4))
        return SWATTN_ERR_ALIGN;
    if (d->k_scale && (!aligned(d->k_scale, 4) || !aligned(d->v_scale, 4))) return SWATTN_ERR_ALIGN;
    if (!std::isfinite(scale)) return SWATTN_ERR_ARG;

    const int64_t G = d->num_heads / d->num_kv_heads;
    const int64_t R = (int64_t)n_q * G;
    const int64_t n_elems = (int64_t)d->batch * n_q * d->num_heads * d->head_dim;
    // q and out must not overlap.
    {
        const uintptr_t q0 = reinterpret_cast<uintptr_t>(q);
        const uintptr_t q1 = q0 + (uintptr_t)(n_elems * dtype_bytes(d->q_dtype));
        const uintptr_t o0 = reinterpret_cast<uintptr_t>(out);
        const uintptr_t o1 = o0 + (uintptr_t)(n_elems * dtype_bytes(d->out_dtype));
        if (q0 < o1 && o0 < q1) return SWATTN_ERR_ARG;
    }
    float* ws_o = nullptr;
    float* ws_lse = nullptr;
    int32_t* counters = nullptr;
    if (plan.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < plan.workspace_bytes) return SWATTN_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return SWATTN_ERR_ALIGN;
        const int64_t rows_total = (int64_t)d->batch * d->num_kv_heads * R;
        const int64_t o_bytes = ((rows_total * plan.num_splits * d->head_dim * 4) + 255) / 256 * 256;
        char* base = reinterpret_cast<char*>(workspace);
        if (plan.fused_merge) counters = reinterpret_cast<int32_t*>(base);
        ws_o = reinterpret_cast<float*>(base + SWATTN_WORKSPACE_COUNTER_BYTES);
        ws_lse = reinterpret_cast<float*>(base + SWATTN_WORKSPACE_COUNTER_BYTES + o_bytes);
    }

    PartitionParams& p = call->p;
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.block_table = block_table;
    p.ctx_len = ctx_len;
    p.k_scale = d->k_scale;
    p.v_scale = d->v_scale;
    p.out = out;
    p.ws_o = ws_o;
    p.ws_lse = ws_lse;
    p.counters = counters;
    p.k_new = nullptr;
    p.v_new = nullptr;
    p.k_dst = nullptr;
    p.v_dst = nullptr;
    p.B = d->batch;
    p.H = d->num_heads;
    p.Hkv = d->num_kv_heads;
    p.G = (int32_t)G;
    p.D = d->head_dim;
    p.bs = d->block_size;
    p.bs_log2 = -1;
    for (int k = 0; k < 31; ++k)
        if (d->block_size == (1 << k)) p.bs_log2 = k;
    p.max_blocks = d->max_blocks_per_seq;
    p.num_blocks = d->num_blocks;
    p.n_q = n_q;
    p.window = window;
    p.R = (int32_t)R;
    p.max_ctx = d->max_ctx_len;
    p.S = plan.num_splits;
    p.rows_per_chunk = plan.rows_per_chunk;
    p.row_chunks = plan.row_chunks;
    p.col_splits = plan.col_splits;
    p.q_dtype = d->q_dtype;
    p.kv_dtype = d->kv_dtype;
    p.out_dtype = d->out_dtype;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);   // log2(e)
    p.tile_keys = plan.tile_keys;

    MergeParams& m = call->m;
    {
        m.ws_o = ws_o;
        m.ws_lse = ws_lse;
        m.out = out;
        m.B = d->batch;
        m.H = d->num_heads;
        m.Hkv = d->num_kv_heads;
        m.G = (int32_t)G;
        m.D = d->head_dim;
        m.n_q = n_q;
        m.R = (int32_t)R;
        m.S = plan.num_splits;
        m.out_dtype = d->out_dtype;
    }
    return SWATTN_OK;
}

swattn_status_t launch_attend(const AttendCall& call, void* stream) {
    const int err = call.plan.variant == SWATTN_VARIANT_MFMA ? launch_partition_mfma(call.p, call.plan.grid, stream)
                                                             : launch_partition_valu(call.p, call.plan.grid, stream);
    if (err != 0) return SWATTN_ERR_HIP;
    if (call.plan.merge_grid > 0 && launch_merge(call.m, call.plan.merge_grid, stream) != 0) return SWATTN_ERR_HIP;
    return SWATTN_OK;
}


namespace {

// The checks and launch shape of an append call; nothing is enqueued.
swattn_status_t prepare_append(const swattn_desc_t* d, const void* k_new, const void* v_new,
                               swattn_dtype_t new_dtype, const int32_t* block_table, const int32_t* ctx_len,
                               int32_t n_new, void* k_cache, void* v_cache, AppendParams* out, int64_t* grid_out) {
    if (!d) return SWATTN_ERR_NULL;
    if (d->batch < 1 || d->num_kv_heads < 1) return SWATTN_ERR_SHAPE;
    if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return SWATTN_ERR_SHAPE;
    if (d->block_size < 1 || d->max_blocks_per_seq < 1 || d->num_blocks < 1 || d->max_ctx_len < 1)
        return SWATTN_ERR_SHAPE;
    if ((int64_t)d->max_ctx_len > (int64_t)d->max_blocks_per_seq * d->block_size) return SWATTN_ERR_SHAPE;
    if ((int64_t)d->num_blocks * d->num_kv_heads * d->block_size > INT32_MAX) return SWATTN_ERR_SHAPE;
    if ((int64_t)d->max_blocks_per_seq * d->block_size > INT32_MAX) return SWATTN_ERR_SHAPE;
    if (n_new < 1 || n_new > SWATTN_MAX_PREFILL_NQ) return SWATTN_ERR_NQ;
    if (new_dtype != SWATTN_F32 && new_dtype != SWATTN_BF16) return SWATTN_ERR_DTYPE;
    if (d->kv_dtype != SWATTN_F32 && d->kv_dtype != SWATTN_BF16 && d->kv_dtype != SWATTN_FP8_E4M3)
        return SWATTN_ERR_DTYPE;
    const bool fp8 = d->kv_dtype == SWATTN_FP8_E4M3;
    if (fp8 && (!d->k_scale || !d->v_scale)) return SWATTN_ERR_DTYPE;
    if (!fp8 && (d->k_scale || d->v_scale)) return SWATTN_ERR_DTYPE;
    if (!k_new || !v_new || !block_table || !ctx_len || !k_cache || !v_cache) return SWATTN_ERR_NULL;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_table, 4) || !aligned(ctx_len, 4))
        return SWATTN_ERR_ALIGN;
    if (fp8 && (!aligned(d->k_scale, 4) || !aligned(d->v_scale, 4))) return SWATTN_ERR_ALIGN;
    const int64_t threads = 2 * (int64_t)d->batch * n_new * d->num_kv_heads * (d->head_dim / 8);
    const int64_t grid = (threads + kBlockThreads - 1) / kBlockThreads;
    if (grid > INT32_MAX) return SWATTN_ERR_SHAPE;

    AppendParams& p = *out;
    p.k_new = k_new;
    p.v_new = v_new;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_table = block_table;
    p.ctx_len = ctx_len;
    p.k_scale = d->k_scale;
    p.v_scale = d->v_scale;
    p.B = d->batch;
    p.Hkv = d->num_kv_heads;
    p.D = d->head_dim;
    p.bs = d->block_size;
    p.max_blocks = d->max_blocks_per_seq;
    p.num_blocks = d->num_blocks;
    p.max_ctx = d->max_ctx_len;
    p.n_new = n_new;
    p.new_dtype = new_dtype;
    p.kv_dtype = d->kv_dtype;
    *grid_out = grid;
    return SWATTN_OK;
}

}  // namespace

swattn_status_t attend(const swattn_desc_t* d, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* ctx_len, int32_t n_q, int32_t window,
                       float scale, void* out, void* workspace, size_t workspace_bytes, void* stream,
                       int32_t max_nq) {
    AttendCall call;
    const swattn_status_t st = prepare_attend(d, q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale,
                                              out, workspace, workspace_bytes, max_nq, &call);
    return st != SWATTN_OK ? st : launch_attend(call, stream);
}

}  // namespace swattn

extern "C" swattn_status_t swattn_verify(const swattn_desc_t* d, const void* q, const void* k_cache,
                                         const void* v_cache, const int32_t* block_table,
                                         const int32_t* ctx_len, int32_t n_q, int32_t window, float scale,
                                         void* out, void* workspace, size_t workspace_bytes, void* stream) {
    return swattn::attend(d, q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale, out, workspace,
                          workspace_bytes, stream, SWATTN_MAX_NQ);
}

extern "C" swattn_status_t swattn_prefill(const swattn_desc_t* d, const void* q, const void* k_cache,
                                          const void* v_cache, const int32_t* block_table,
                                          const int32_t* ctx_len, int32_t n_q, int32_t window, float scale,
                                          void* out, void* workspace, size_t workspace_bytes, void* stream) {
    return swattn::attend(d, q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale, out, workspace,
                          workspace_bytes, stream, SWATTN_MAX_PREFILL_NQ);
}

extern "C" swattn_status_t swattn_check_inputs(const swattn_desc_t* d, const int32_t* block_table,
                                               const int32_t* ctx_len, int32_t n_q, int32_t window,
                                               void* stream) {
    using namespace swattn;
    swattn_status_t st = validate_desc(d, n_q, window, SWATTN_MAX_PREFILL_NQ);
    if (st != SWATTN_OK) return st;
    if (!block_table || !ctx_len) return SWATTN_ERR_NULL;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    std::vector<int32_t> ctx(d->batch);
    std::vector<int32_t> table((size_t)d->batch * d->max_blocks_per_seq);
    if (hipMemcpyAsync(ctx.data(), ctx_len, ctx.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess)
        return SWATTN_ERR_HIP;
    if (hipMemcpyAsync(table.data(), block_table, table.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess)
        return SWATTN_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SWATTN_ERR_HIP;
    const int64_t cap = (int64_t)d->max_blocks_per_seq * d->block_size;
    for (int b = 0; b < d->batch; ++b)
        if (ctx[b] < n_q || ctx[b] > cap || ctx[b] > d->max_ctx_len) return SWATTN_ERR_CTX;
    for (int b = 0; b < d->batch; ++b) {
        const int64_t lo = std::max<int64_t>(0, (int64_t)ctx[b] - n_q - window + 1);
        const int64_t hi = ctx[b] - 1;
        for (int64_t blk = lo / d->block_size; blk <= hi / d->block_size; ++blk) {
            const int32_t phys = table[(size_t)b * d->max_blocks_per_seq + blk];
            if (phys < 0 || phys >= d->num_blocks) return SWATTN_ERR_BLOCK;
        }
    }
    return SWATTN_OK;
}

extern "C" swattn_status_t swattn_append_kv(const swattn_desc_t* d, const void* k_new, const void* v_new,
                                            swattn_dtype_t new_dtype, const int32_t* block_table,
                                            const int32_t* ctx_len, int32_t n_new, void* k_cache, void* v_cache,
                                            void* stream) {
    using namespace swattn;
    AppendParams p;
    int64_t grid = 0;
    const swattn_status_t st =
        prepare_append(d, k_new, v_new, new_dtype, block_table, ctx_len, n_new, k_cache, v_cache, &p, &grid);
    if (st != SWATTN_OK) return st;
    return launch_kv_append(p, (int)grid, stream) == 0 ? SWATTN_OK : SWATTN_ERR_HIP;
}

extern "C" swattn_status_t swattn_append_verify(const swattn_desc_t* d, const void* q, const void* k_new,
                                                const void* v_new, swattn_dtype_t new_dtype, void* k_cache,
                                                void* v_cache, const int32_t* block_table, const int32_t* ctx_len,
                                                int32_t n_q, int32_t window, float scale, void* out,
                                                void* workspace, size_t workspace_bytes, void* stream) {
    using namespace swattn;
    AppendParams ap;
    int64_t agrid = 0;
    swattn_status_t st =
        prepare_append(d, k_new, v_new, new_dtype, block_table, ctx_len, n_q, k_cache, v_cache, &ap, &agrid);
    if (st != SWATTN_OK) return st;
    AttendCall call;
    st = prepare_attend(d, q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale, out, workspace,
                        workspace_bytes, SWATTN_MAX_NQ, &call);
    if (st != SWATTN_OK) return st;
    // One launch where the matrix-core kernel can take the new rows as they are (bfloat16
    // rows into a bfloat16 cache: the append is a copy): it reads the keys at the new
    // positions from k_new / v_new and writes them into the cache itself.  Otherwise
    // the append kernel, then the attention call.
    if (call.plan.variant == SWATTN_VARIANT_MFMA && new_dtype == SWATTN_BF16 && d->kv_dtype == SWATTN_BF16) {
        call.p.k_new = k_new;
        call.p.v_new = v_new;
        call.p.k_dst = k_cache;
        call.p.v_dst = v_cache;
        return launch_attend(call, stream);
    }
    if (launch_kv_append(ap, (int)agrid, stream) != 0) return SWATTN_ERR_HIP;
    return launch_attend(call, stream);
}

namespace swattn {
namespace {

swattn_status_t accept_shape(int32_t batch, int32_t n_q, int32_t vocab, int64_t* nchunk, size_t* bytes) {
    if (batch < 1 || vocab < 1) return SWATTN_ERR_SHAPE;
    if (n_q < 1 || n_q > SWATTN_MAX_NQ) return SWATTN_ERR_NQ;
    const int64_t nc = ((int64_t)vocab + kAcceptChunk - 1) / kAcceptChunk;
    if ((int64_t)batch * n_q * nc > INT32_MAX) return SWATTN_ERR_SHAPE;
    *nchunk = nc;
    *bytes = (size_t)((int64_t)batch * n_q * nc * 8);
    return SWATTN_OK;
}

}  // namespace
}  // namespace swattn

extern "C" swattn_status_t swattn_workspace_init(void* workspace, size_t bytes, void* stream) {
    if (!workspace) return SWATTN_ERR_NULL;
    if (!swattn::aligned(workspace, 16)) return SWATTN_ERR_ALIGN;
    const size_t n = (bytes < SWATTN_WORKSPACE_COUNTER_BYTES ? bytes : SWATTN_WORKSPACE_COUNTER_BYTES) / 4;
    return swattn::launch_zero_words(reinterpret_cast<int32_t*>(workspace), (int)n, stream) == 0 ? SWATTN_OK
                                                                                                : SWATTN_ERR_HIP;
}

extern "C" swattn_status_t swattn_greedy_accept_workspace(int32_t batch, int32_t n_q, int32_t vocab,
                                                          size_t* bytes) {
    if (!bytes) return SWATTN_ERR_NULL;
    int64_t nc;
    size_t b;
    const swattn_status_t st = swattn::accept_shape(batch, n_q, vocab, &nc, &b);
    if (st == SWATTN_OK) *bytes = b;
    return st;
}

extern "C" swattn_status_t swattn_greedy_accept(const void* logits, swattn_dtype_t logits_dtype, int32_t batch,
                                                int32_t n_q, int32_t vocab, const int32_t* draft_ids,
                                                int32_t* target_ids, int32_t* accepted, int32_t* next_token,
                                                void* workspace, size_t workspace_bytes, void* stream) {
    using namespace swattn;
    int64_t nchunk;
    size_t need;
    swattn_status_t st = accept_shape(batch, n_q, vocab, &nchunk, &need);
    if (st != SWATTN_OK) return st;
    if (logits_dtype != SWATTN_F32 && logits_dtype != SWATTN_BF16) return SWATTN_ERR_DTYPE;
    if (!logits || !target_ids || !accepted || !next_token || (n_q > 1 && !draft_ids)) return SWATTN_ERR_NULL;
    if (!workspace || workspace_bytes < need) return SWATTN_ERR_WORKSPACE;
    const uintptr_t elt = logits_dtype == SWATTN_F32 ? 4 : 2;
    if (!aligned(logits, elt) || !aligned(workspace, 8) || !aligned(target_ids, 4) || !aligned(accepted, 4) ||
        !aligned(next_token, 4) || (draft_ids && !aligned(draft_ids, 4)))
        return SWATTN_ERR_ALIGN;
    AcceptParams p;
    p.logits = logits;
    p.draft_ids = draft_ids;
    p.target_ids = target_ids;
    p.accepted = accepted;
    p.next_token = next_token;
    p.partial = reinterpret_cast<uint64_t*>(workspace);
    p.B = batch;
    p.n_q = n_q;
    p.vocab = vocab;
    p.nchunk = (int32_t)nchunk;
    p.logits_dtype = logits_dtype;
    // 16-byte loads when every row starts 16-byte aligned
    const int64_t per_load = 16 / (int64_t)elt;
    p.vec_ok = aligned(logits, 16) && vocab % per_load == 0;
    const int64_t grid1 = (int64_t)batch * n_q * nchunk;
    return launch_accept(p, (int)grid1, stream) == 0 ? SWATTN_OK : SWATTN_ERR_HIP;
}
