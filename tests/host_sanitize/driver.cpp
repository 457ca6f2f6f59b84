// Host-side checks of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Built with g++ (no GPU code) from plan.cpp and api.cpp, with the kernel launchers
// replaced by the stubs below, which check what a launch would receive and record
// it.  Every entry point's host path runs: planning over a sweep of shapes, every
// host-checkable error, and well-formed calls with fake (aligned, never
// dereferenced) device pointers, whose launch parameters are checked against the
// plan.  Prints "ok <cases>" and exits 0, or prints the first mismatch and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>

#include "swattn.h"
#include "swattn_internal.h"

namespace swattn {

struct Recorded {
    int partition_mfma = 0, partition_valu = 0, merge = 0, zero = 0, append = 0, accept = 0;
    PartitionParams p{};
    MergeParams m{};
    int grid = 0, merge_grid = 0;
} g_rec;

static bool g_fail = false;
#define CHECK(cond)                                                                 \
    do {                                                                            \
        if (!(cond)) {                                                              \
            std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);            \
            g_fail = true;                                                          \
        }                                                                           \
    } while (0)

// Stub launchers: consistency of what a kernel would receive.
int launch_partition_mfma(const PartitionParams& p, int grid, void*) {
    ++g_rec.partition_mfma;
    g_rec.p = p;
    g_rec.grid = grid;
    CHECK(grid == p.B * p.Hkv * p.row_chunks * p.col_splits * p.S);
    CHECK(p.rows_per_chunk == 16 || p.rows_per_chunk == 32 || p.rows_per_chunk == 64);
    if (p.rows_per_chunk == 64) CHECK(p.col_splits == 1 && p.kv_dtype == SWATTN_BF16);
    CHECK(p.col_splits == 1 || p.col_splits == 2 || p.col_splits == 4);
    CHECK(p.tile_keys == 32 || p.tile_keys == 64);
    CHECK(p.row_chunks == (p.R + p.rows_per_chunk - 1) / p.rows_per_chunk);
    CHECK(p.S >= 1);
    CHECK((p.S > 1) == (p.ws_o != nullptr));
    return 0;
}
int launch_partition_valu(const PartitionParams& p, int grid, void*) {
    ++g_rec.partition_valu;
    g_rec.p = p;
    g_rec.grid = grid;
    CHECK(grid == p.B * p.Hkv * p.row_chunks * p.S);
    CHECK(p.col_splits == 1);
    return 0;
}
int launch_merge(const MergeParams& m, int grid, void*) {
    ++g_rec.merge;
    g_rec.m = m;
    g_rec.merge_grid = grid;
    CHECK(grid >= 1 && m.S > 1);
    return 0;
}
int launch_zero_words(int32_t* w, int n, void*) {
    ++g_rec.zero;
    CHECK(w != nullptr && n >= 0 && n <= SWATTN_WORKSPACE_COUNTER_BYTES / 4);
    return 0;
}
int launch_kv_append(const AppendParams& p, int grid, void*) {
    ++g_rec.append;
    CHECK(grid >= 1 && p.n_new >= 1);
    return 0;
}
int launch_accept(const AcceptParams& p, int grid1, void*) {
    ++g_rec.accept;
    CHECK(grid1 == p.B * p.n_q * p.nchunk);
    return 0;
}

}  // namespace swattn

using namespace swattn;

// fake device pointers: 256-byte aligned addresses in distinct ranges, never dereferenced
static void* fake(uintptr_t k) { return reinterpret_cast<void*>((uintptr_t)0x10000000000ull * (k + 1)); }

static swattn_desc_t base_desc() {
    swattn_desc_t d;
    std::memset(&d, 0, sizeof d);
    d.batch = 24;
    d.num_heads = 8;
    d.num_kv_heads = 2;
    d.head_dim = 256;
    d.block_size = 16;
    d.max_blocks_per_seq = 256;
    d.num_blocks = 6144;
    d.max_ctx_len = 4096;
    d.q_dtype = SWATTN_BF16;
    d.kv_dtype = SWATTN_BF16;
    d.out_dtype = SWATTN_BF16;
    return d;
}

static int g_cases = 0;

static swattn_status_t verify(const swattn_desc_t& d, int n_q, int window, void* ws, size_t ws_bytes) {
    ++g_cases;
    return swattn_verify(&d, fake(0), fake(1), fake(2), (const int32_t*)fake(3), (const int32_t*)fake(4), n_q, window,
                         0.0625f, fake(5), ws, ws_bytes, nullptr);
}

int main() {
    // ---- every status code has a description
    for (int s = 0; s >= -12; --s) CHECK(std::strlen(swattn_status_str((swattn_status_t)s)) > 0);
    CHECK(swattn_abi_version() == SWATTN_ABI_VERSION);

    // ---- host-checkable errors
    swattn_desc_t d = base_desc();
    swattn_plan_t plan;
    CHECK(swattn_plan(nullptr, 8, 188, &plan) == SWATTN_ERR_NULL);
    CHECK(swattn_plan(&d, 8, 188, nullptr) == SWATTN_ERR_NULL);
    CHECK(swattn_plan(&d, 0, 188, &plan) == SWATTN_ERR_NQ);
    CHECK(swattn_plan(&d, 65, 188, &plan) == SWATTN_ERR_NQ);
    CHECK(swattn_prefill_plan(&d, 512, 188, &plan) == SWATTN_OK);
    CHECK(swattn_prefill_plan(&d, 513, 188, &plan) == SWATTN_ERR_NQ);
    CHECK(swattn_plan(&d, 8, 0, &plan) == SWATTN_ERR_WINDOW);
    {
        swattn_desc_t e = d;
        e.num_heads = 7;
        CHECK(swattn_plan(&e, 8, 188, &plan) == SWATTN_ERR_SHAPE);
        e = d;
        e.head_dim = 96;
        CHECK(swattn_plan(&e, 8, 188, &plan) == SWATTN_ERR_SHAPE);
        e = d;
        e.max_ctx_len = 4097;
        CHECK(swattn_plan(&e, 8, 188, &plan) == SWATTN_ERR_SHAPE);
        e = d;
        e.kv_dtype = SWATTN_FP8_E4M3;
        CHECK(swattn_plan(&e, 8, 188, &plan) == SWATTN_ERR_DTYPE);     // no scales
        e.k_scale = (const float*)fake(6);
        e.v_scale = (const float*)fake(7);
        CHECK(swattn_plan(&e, 8, 188, &plan) == SWATTN_OK);
        e = d;
        e.num_splits = -1;
        CHECK(swattn_plan(&e, 8, 188, &plan) == SWATTN_ERR_ARG);
        e = d;
        e.rows_per_chunk = 8;
        CHECK(swattn_plan(&e, 8, 188, &plan) == SWATTN_ERR_ARG);
        e = d;
        e.col_splits = 3;
        CHECK(swattn_plan(&e, 8, 188, &plan) == SWATTN_ERR_ARG);
        e = d;
        e.variant = SWATTN_VARIANT_VALU;
        e.col_splits = 2;
        CHECK(swattn_plan(&e, 8, 188, &plan) == SWATTN_ERR_ARG);
        e = d;
        e.batch = 1;
        e.merge = SWATTN_MERGE_FUSED;
        e.num_splits = 3;
        CHECK(swattn_plan(&e, 8, 188, &plan) == SWATTN_OK && plan.fused_merge == 1);
        e.batch = 100000;
        CHECK(swattn_plan(&e, 8, 188, &plan) == SWATTN_ERR_SHAPE);    // more merge groups than counters
    }
    CHECK(verify(d, 8, 188, nullptr, 0) == SWATTN_OK);
    CHECK(g_rec.partition_mfma == 1 && g_rec.merge == 0);
    {
        ++g_cases;
        CHECK(swattn_verify(&d, nullptr, fake(1), fake(2), (const int32_t*)fake(3), (const int32_t*)fake(4), 8, 188,
                            0.0625f, fake(5), nullptr, 0, nullptr) == SWATTN_ERR_NULL);
        CHECK(swattn_verify(&d, (char*)fake(0) + 2, fake(1), fake(2), (const int32_t*)fake(3), (const int32_t*)fake(4), 8,
                            188, 0.0625f, fake(5), nullptr, 0, nullptr) == SWATTN_ERR_ALIGN);
        CHECK(swattn_verify(&d, fake(0), fake(1), fake(2), (const int32_t*)fake(3), (const int32_t*)fake(4), 8, 188,
                            0.0625f, fake(0), nullptr, 0, nullptr) == SWATTN_ERR_ARG);      // out aliases q
        CHECK(swattn_verify(&d, fake(0), fake(1), fake(2), (const int32_t*)fake(3), (const int32_t*)fake(4), 8, 188,
                            1.0f / 0.0f, fake(5), nullptr, 0, nullptr) == SWATTN_ERR_ARG);   // scale not finite
        swattn_desc_t e = d;
        e.num_splits = 4;
        CHECK(swattn_plan(&e, 8, 188, &plan) == SWATTN_OK && plan.workspace_bytes > 0);
        CHECK(verify(e, 8, 188, nullptr, 0) == SWATTN_ERR_WORKSPACE);
        CHECK(verify(e, 8, 188, fake(8), plan.workspace_bytes - 1) == SWATTN_ERR_WORKSPACE);
        const int before = g_rec.partition_mfma;
        CHECK(verify(e, 8, 188, fake(8), plan.workspace_bytes) == SWATTN_OK);
        CHECK(g_rec.partition_mfma == before + 1 && g_rec.p.S == 4);
    }

    // ---- a sweep of shapes through plan + verify: every plan launches consistently
    std::mt19937 rng(12345);
    auto pick = [&](std::initializer_list<int> v) { return *(v.begin() + rng() % v.size()); };
    for (int it = 0; it < 4000; ++it) {
        swattn_desc_t e = base_desc();
        e.batch = pick({1, 2, 3, 8, 24, 48, 96, 256, 1000});
        e.num_kv_heads = pick({1, 2, 4});
        e.num_heads = e.num_kv_heads * pick({1, 2, 4, 8, 16});
        e.head_dim = pick({64, 128, 256});
        e.block_size = pick({1, 16, 300});
        e.max_ctx_len = pick({1, 64, 300, 1000, 4096});
        e.max_blocks_per_seq = (e.max_ctx_len + e.block_size - 1) / e.block_size + pick({0, 1});
        e.num_blocks = e.batch * e.max_blocks_per_seq;
        const int dt = pick({0, 1, 2, 3});
        e.q_dtype = dt == 3 ? SWATTN_F32 : SWATTN_BF16;
        e.kv_dtype = dt == 0 ? SWATTN_BF16 : dt == 1 ? SWATTN_FP8_E4M3 : SWATTN_F32;
        e.out_dtype = pick({0, 1}) ? SWATTN_F32 : SWATTN_BF16;
        if (e.kv_dtype == SWATTN_FP8_E4M3) {
            e.k_scale = (const float*)fake(6);
            e.v_scale = (const float*)fake(7);
        }
        e.num_splits = pick({0, 0, 1, 2, 5});
        e.merge = pick({0, 0, 1, 2});
        if (e.head_dim == 256 && e.q_dtype == SWATTN_BF16 && e.kv_dtype != SWATTN_F32) {
            e.rows_per_chunk = pick({0, 0, 16, 32});
            e.col_splits = pick({0, 0, 1, 2, 4});
        }
        const int n_q = pick({1, 2, 8, 17, 64, 65, 512});
        const int window = pick({1, 16, 188, 4096});
        const bool prefill = n_q > SWATTN_MAX_NQ;
        swattn_plan_t pl;
        const swattn_status_t st = prefill ? swattn_prefill_plan(&e, n_q, window, &pl) : swattn_plan(&e, n_q, window, &pl);
        if (st != SWATTN_OK) {
            CHECK(st == SWATTN_ERR_CTX || st == SWATTN_ERR_SHAPE || st == SWATTN_ERR_ARG || st == SWATTN_ERR_DTYPE);
            continue;
        }
        CHECK(pl.grid >= 1 && pl.num_splits >= 1 && pl.row_chunks >= 1);
        CHECK((pl.num_splits > 1) == (pl.workspace_bytes > 0));
        CHECK(pl.fused_merge == 0 || pl.merge_grid == 0);
        const int m0 = g_rec.partition_mfma + g_rec.partition_valu, k0 = g_rec.merge;
        ++g_cases;
        const swattn_status_t vs =
            (prefill ? swattn_prefill : swattn_verify)(&e, fake(0), fake(1), fake(2), (const int32_t*)fake(3),
                                                       (const int32_t*)fake(4), n_q, window, 0.125f, fake(5),
                                                       pl.workspace_bytes ? fake(8) : nullptr, pl.workspace_bytes,
                                                       nullptr);
        CHECK(vs == SWATTN_OK);
        CHECK(g_rec.partition_mfma + g_rec.partition_valu == m0 + 1);
        CHECK(g_rec.merge == k0 + (pl.merge_grid > 0 ? 1 : 0));
        CHECK(g_rec.grid == pl.grid);
        CHECK(g_rec.p.S == pl.num_splits && g_rec.p.col_splits == pl.col_splits);
        CHECK((g_rec.p.counters != nullptr) == (pl.fused_merge == 1));
    }

    // ---- the other entry points' host paths
    {
        size_t bytes = 0;
        CHECK(swattn_workspace_bytes(&d, 8, 188, &bytes) == SWATTN_OK && bytes == 0);
        CHECK(swattn_workspace_bytes(&d, 8, 188, nullptr) == SWATTN_ERR_NULL);
        CHECK(swattn_workspace_init(nullptr, 16, nullptr) == SWATTN_ERR_NULL);
        CHECK(swattn_workspace_init(fake(8), 1 << 20, nullptr) == SWATTN_OK && g_rec.zero == 1);
        CHECK(swattn_append_kv(&d, fake(0), fake(1), SWATTN_BF16, (const int32_t*)fake(3), (const int32_t*)fake(4), 8,
                               fake(5), fake(6), nullptr) == SWATTN_OK && g_rec.append == 1);
        CHECK(swattn_append_kv(&d, fake(0), fake(1), SWATTN_FP8_E4M3, (const int32_t*)fake(3), (const int32_t*)fake(4),
                               8, fake(5), fake(6), nullptr) == SWATTN_ERR_DTYPE);
        CHECK(swattn_append_kv(&d, fake(0), fake(1), SWATTN_BF16, (const int32_t*)fake(3), (const int32_t*)fake(4), 0,
                               fake(5), fake(6), nullptr) == SWATTN_ERR_NQ);
        const int m0 = g_rec.partition_mfma;
        CHECK(swattn_append_verify(&d, fake(0), fake(9), fake(10), SWATTN_BF16, fake(1), fake(2), (const int32_t*)fake(3),
                                   (const int32_t*)fake(4), 8, 188, 0.0625f, fake(5), nullptr, 0, nullptr) == SWATTN_OK);
        CHECK(g_rec.partition_mfma == m0 + 1 && g_rec.p.k_new == fake(9) && g_rec.append == 1);   // one launch
        swattn_desc_t e = d;
        e.kv_dtype = SWATTN_FP8_E4M3;
        e.k_scale = (const float*)fake(6);
        e.v_scale = (const float*)fake(7);
        CHECK(swattn_append_verify(&e, fake(0), fake(9), fake(10), SWATTN_BF16, fake(1), fake(2), (const int32_t*)fake(3),
                                   (const int32_t*)fake(4), 8, 188, 0.0625f, fake(5), nullptr, 0, nullptr) == SWATTN_OK);
        CHECK(g_rec.append == 2 && g_rec.p.k_new == nullptr);                                    // append kernel first
        size_t acc_bytes = 0;
        CHECK(swattn_greedy_accept_workspace(1, 8, 262144, &acc_bytes) == SWATTN_OK && acc_bytes > 0);
        CHECK(swattn_greedy_accept_workspace(1, 0, 262144, &acc_bytes) == SWATTN_ERR_NQ);
        CHECK(swattn_greedy_accept(fake(0), SWATTN_BF16, 1, 8, 262144, (const int32_t*)fake(1), (int32_t*)fake(2),
                                   (int32_t*)fake(3), (int32_t*)fake(4), fake(5), acc_bytes, nullptr) == SWATTN_OK);
        CHECK(g_rec.accept == 1);
        CHECK(swattn_greedy_accept(fake(0), SWATTN_BF16, 1, 8, 262144, nullptr, (int32_t*)fake(2), (int32_t*)fake(3),
                                   (int32_t*)fake(4), fake(5), acc_bytes, nullptr) == SWATTN_ERR_NULL);
        CHECK(swattn_greedy_accept(fake(0), SWATTN_BF16, 1, 8, 262144, (const int32_t*)fake(1), (int32_t*)fake(2),
                                   (int32_t*)fake(3), (int32_t*)fake(4), fake(5), acc_bytes - 1,
                                   nullptr) == SWATTN_ERR_WORKSPACE);
        CHECK(swattn_check_inputs(nullptr, nullptr, nullptr, 8, 188, nullptr) == SWATTN_ERR_NULL);
        CHECK(swattn_check_inputs(&d, nullptr, (const int32_t*)fake(4), 8, 188, nullptr) == SWATTN_ERR_NULL);
        g_cases += 16;
    }

    if (g_fail) return 1;
    std::printf("ok %d\n", g_cases);
    return 0;
}
