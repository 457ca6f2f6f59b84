"""CPU tests of the C ABI: the library loads, exports what include/swattn.h
declares, and the host-side planner / argument checks behave (no GPU needed:
none of these calls reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import speculative_verify_kv_amd as sw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "swattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swattn_[a-z_]+)\s*\(", text)))


def test_library_exports_every_header_symbol():
    names = header_functions()
    assert names == sorted(sw.EXPORTED)
    lib = sw.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert callable(getattr(sw, n)), n      # binding uses the same names


def test_abi_version_and_status_strings():
    assert sw.swattn_abi_version() == sw.ABI_VERSION == 3
    for code in sw.STATUS:
        s = sw.swattn_status_str(code)
        assert s and s != "unknown status"
    assert sw.swattn_status_str(12345) == "unknown status"


def desc(**kw):
    d = sw.swattn_desc_t()
    base = dict(batch=24, num_heads=8, num_kv_heads=2, head_dim=256, block_size=16,
                max_blocks_per_seq=256, num_blocks=6144, max_ctx_len=4096,
                q_dtype=sw.SWATTN_BF16, kv_dtype=sw.SWATTN_BF16, out_dtype=sw.SWATTN_BF16,
                k_scale=None, v_scale=None, num_splits=0, variant=0, merge=0)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


def status(d, n_q=8, window=188):
    st, _ = sw.swattn_plan(d, n_q, window, check=False)
    return sw.STATUS[st]


@pytest.mark.parametrize("kw,n_q,window,expect", [
    (dict(batch=0), 8, 188, "SWATTN_ERR_SHAPE"),
    (dict(num_heads=6, num_kv_heads=4), 8, 188, "SWATTN_ERR_SHAPE"),
    (dict(head_dim=96), 8, 188, "SWATTN_ERR_SHAPE"),
    (dict(head_dim=512), 8, 188, "SWATTN_ERR_SHAPE"),
    (dict(block_size=0), 8, 188, "SWATTN_ERR_SHAPE"),
    (dict(num_blocks=0), 8, 188, "SWATTN_ERR_SHAPE"),
    (dict(max_ctx_len=4097), 8, 188, "SWATTN_ERR_SHAPE"),
    (dict(), 0, 188, "SWATTN_ERR_NQ"),
    (dict(), 65, 188, "SWATTN_ERR_NQ"),
    (dict(), 8, 0, "SWATTN_ERR_WINDOW"),
    (dict(max_ctx_len=7), 8, 188, "SWATTN_ERR_CTX"),
    (dict(q_dtype=sw.SWATTN_FP8_E4M3), 8, 188, "SWATTN_ERR_DTYPE"),
    (dict(out_dtype=sw.SWATTN_FP8_E4M3), 8, 188, "SWATTN_ERR_DTYPE"),
    (dict(kv_dtype=7), 8, 188, "SWATTN_ERR_DTYPE"),
    (dict(kv_dtype=sw.SWATTN_FP8_E4M3), 8, 188, "SWATTN_ERR_DTYPE"),          # no scales
    (dict(k_scale=16, v_scale=32), 8, 188, "SWATTN_ERR_DTYPE"),               # scales without e4m3
    (dict(variant=sw.SWATTN_VARIANT_MFMA, q_dtype=sw.SWATTN_F32), 8, 188, "SWATTN_ERR_DTYPE"),
    (dict(variant=sw.SWATTN_VARIANT_MFMA, kv_dtype=sw.SWATTN_F32), 8, 188, "SWATTN_ERR_DTYPE"),
    (dict(variant=9), 8, 188, "SWATTN_ERR_ARG"),
    (dict(num_splits=-1), 8, 188, "SWATTN_ERR_ARG"),
    (dict(merge=3), 8, 188, "SWATTN_ERR_ARG"),
    (dict(merge=-1), 8, 188, "SWATTN_ERR_ARG"),
    # chunk-geometry overrides: 16 / 64-row chunks and column splits need head_dim 256;
    # 64-row chunks are for bfloat16 caches and take no column split
    (dict(rows_per_chunk=48), 8, 188, "SWATTN_ERR_ARG"),
    (dict(col_splits=3), 8, 188, "SWATTN_ERR_ARG"),
    (dict(rows_per_chunk=16, head_dim=128), 8, 188, "SWATTN_ERR_ARG"),
    (dict(rows_per_chunk=64, head_dim=128), 8, 188, "SWATTN_ERR_ARG"),
    (dict(rows_per_chunk=64, col_splits=2), 8, 188, "SWATTN_ERR_ARG"),
    (dict(rows_per_chunk=64, kv_dtype=sw.SWATTN_FP8_E4M3, k_scale=16, v_scale=32), 8, 188, "SWATTN_ERR_ARG"),
    (dict(rows_per_chunk=64, variant=sw.SWATTN_VARIANT_VALU), 8, 188, "SWATTN_ERR_ARG"),
    (dict(rows_per_chunk=64), 8, 188, "SWATTN_OK"),
    (dict(rows_per_chunk=16, col_splits=4), 8, 188, "SWATTN_OK"),
    (dict(), 8, 188, "SWATTN_OK"),
    (dict(), 64, 188, "SWATTN_OK"),
    (dict(), 1, 2 ** 31 - 1, "SWATTN_OK"),
])
def test_plan_validation(kw, n_q, window, expect):
    assert status(desc(**kw), n_q, window) == expect


def test_tall_chunks_keep_each_split_within_the_key_table():
    # 16 queries x 4 heads in one 64-row chunk scan W + 15 keys: past 512 at W = 500,
    # so the 64-row plan splits in two where 32-row chunks (W + 7 keys) need none (1024
    # units fill the CUs: no split for idle CUs)
    p = sw.swattn_plan(desc(batch=256), 16, 500)
    assert p.rows_per_chunk == 64 and p.num_splits == 2 and p.tile_keys == 32
    p = sw.swattn_plan(desc(batch=256, rows_per_chunk=32), 16, 500)
    assert p.rows_per_chunk == 32 and p.num_splits == 1
    assert sw.swattn_plan(desc(batch=256), 16, 497).num_splits == 1


def test_plan_null_pointers():
    lib = sw.lib()
    p = sw.swattn_plan_t()
    assert lib.swattn_plan(None, 8, 188, ctypes.byref(p)) == -1
    d = desc()
    assert lib.swattn_plan(ctypes.byref(d), 8, 188, None) == -1
    assert lib.swattn_workspace_bytes(ctypes.byref(d), 8, 188, None) == -1


def test_plan_variants_and_workspace():
    # verify step: 8 queries x GQA 4 = 32 rows -> matrix cores; 48 units leave most CUs
    # idle, so each 32-row chunk becomes two 16-row chunks, each run by two workgroups
    # (output column halves): 192 workgroups
    p = sw.swattn_plan(desc(), 8, 188)
    assert p.variant == sw.SWATTN_VARIANT_MFMA and p.rows_per_chunk == 16 and p.row_chunks == 2
    assert p.grid == 24 * 2 * 2 * 2 * p.num_splits
    R, D, units = 32, 256, 24 * 2
    # split plans: [counters][partial outputs][partial log2-sum-exps]; the partition
    # kernel combines the partials itself, or a merge kernel does when asked to
    for S in (2, 5):
        for variant in (sw.SWATTN_VARIANT_MFMA, sw.SWATTN_VARIANT_VALU):
            for merge in (sw.SWATTN_MERGE_AUTO, sw.SWATTN_MERGE_FUSED, sw.SWATTN_MERGE_KERNEL):
                p = sw.swattn_plan(desc(num_splits=S, variant=variant, merge=merge), 8, 188)
                o_bytes = -(-(units * R * S * D * 4) // 256) * 256
                assert p.num_splits == S and p.variant == variant
                assert p.workspace_bytes == sw.SWATTN_WORKSPACE_COUNTER_BYTES + o_bytes + units * R * S * 4
                # automatic: fused only when a chunk's partials (rows x D x S x 4 B) fit 16 KiB
                rows = 32 if variant == sw.SWATTN_VARIANT_MFMA else 8
                small = rows * D * S * 4 <= 16 * 1024
                if merge == sw.SWATTN_MERGE_FUSED or (merge == sw.SWATTN_MERGE_AUTO and small):
                    assert p.fused_merge == 1 and p.merge_grid == 0
                else:
                    assert p.fused_merge == 0 and p.merge_grid == -(-(units * R) // (1024 // D))
    # decode-sized chunks: 2 rows x D 64 x 3 splits x 4 B = 1.5 KiB -> fused automatically,
    # on the vector ALUs (float32 data) and on the matrix cores (bfloat16)
    tiny = dict(head_dim=64, num_heads=2, num_kv_heads=1, batch=1, num_splits=3)
    f32 = dict(q_dtype=sw.SWATTN_F32, kv_dtype=sw.SWATTN_F32, out_dtype=sw.SWATTN_F32)
    p = sw.swattn_plan(desc(**tiny, **f32), 1, 188)
    assert p.variant == sw.SWATTN_VARIANT_VALU and p.fused_merge == 1 and p.merge_grid == 0
    p = sw.swattn_plan(desc(**tiny), 1, 188)
    assert p.variant == sw.SWATTN_VARIANT_MFMA and p.fused_merge == 1 and p.merge_grid == 0
    # more row chunks than counters: a merge kernel, and a forced fused merge is refused
    many = dict(batch=600, max_blocks_per_seq=16, max_ctx_len=256, num_splits=2)
    p = sw.swattn_plan(desc(**many), 8, 188)
    assert p.num_splits == 2 and p.fused_merge == 0 and p.merge_grid > 0
    assert status(desc(merge=sw.SWATTN_MERGE_FUSED, **many)) == "SWATTN_ERR_SHAPE"
    assert sw.swattn_plan(desc(merge=sw.SWATTN_MERGE_FUSED, **dict(many, batch=512)), 8, 188).fused_merge == 1
    assert sw.swattn_workspace_bytes(desc(), 8, 188) == sw.swattn_plan(desc(), 8, 188).workspace_bytes
    # decode: 4 rows, bfloat16 -> matrix cores (a padded 16-row tile); float32 Q -> vector ALU
    p = sw.swattn_plan(desc(), 1, 188)
    assert p.variant == sw.SWATTN_VARIANT_MFMA and p.rows_per_chunk == 16 and p.num_splits == 1
    p = sw.swattn_plan(desc(kv_dtype=sw.SWATTN_FP8_E4M3, k_scale=16, v_scale=16), 1, 188)
    assert p.variant == sw.SWATTN_VARIANT_MFMA
    p = sw.swattn_plan(desc(q_dtype=sw.SWATTN_F32), 1, 188)
    assert p.variant == sw.SWATTN_VARIANT_VALU
    # float32 data -> vector ALU whatever the row count
    p = sw.swattn_plan(desc(q_dtype=sw.SWATTN_F32, kv_dtype=sw.SWATTN_F32), 64, 188)
    assert p.variant == sw.SWATTN_VARIANT_VALU and p.row_chunks == 64 * 4 // 8
    # 64 queries x 4 = 256 rows -> four 64-row chunks (bfloat16 caches),
    # eight 32-row chunks for E4M3 caches
    p = sw.swattn_plan(desc(), 64, 188)
    assert p.rows_per_chunk == 64 and p.row_chunks == 4 and p.col_splits == 1
    # 192 workgroups fit the CUs: 64-key tiles (one workgroup of eight waves per CU);
    # beyond the CUs, 32-key tiles (two workgroups of four waves per CU)
    assert p.tile_keys == 64 and p.grid == 192
    assert sw.swattn_plan(desc(batch=40), 64, 188).tile_keys == 32
    p = sw.swattn_plan(desc(kv_dtype=sw.SWATTN_FP8_E4M3, k_scale=16, v_scale=32), 64, 188)
    assert p.rows_per_chunk == 32 and p.row_chunks == 8
    # forced split count is honoured (within the chunk count), S = 1 needs no workspace
    p = sw.swattn_plan(desc(num_splits=1), 8, 188)
    assert p.num_splits == 1 and p.workspace_bytes == 0 and p.merge_grid == 0 and p.fused_merge == 0
    p = sw.swattn_plan(desc(num_splits=3), 8, 188)
    assert p.num_splits == 3 and p.workspace_bytes > 0
    p = sw.swattn_plan(desc(num_splits=1000), 8, 188)
    assert p.num_splits == -(-195 // 16)                 # at most one split per 16 keys
    # the matrix-core kernel holds at most 512 keys per workgroup
    p = sw.swattn_plan(desc(num_splits=1), 8, 4096)
    assert p.variant == sw.SWATTN_VARIANT_MFMA and p.num_splits == 8
    # the VALU kernel holds at most 256 keys per workgroup
    p = sw.swattn_plan(desc(variant=sw.SWATTN_VARIANT_VALU, num_splits=1, max_ctx_len=4096), 8, 4096)
    assert p.num_splits == 16


def test_prefill_plan_caps_and_per_chunk_keys():
    # n_q above 64 is for the prefill entry points only; 512 is their cap
    assert sw.swattn_plan(desc(), 65, 188, check=False)[0] == -3
    assert sw.swattn_prefill_plan(desc(), 65, 188).variant == sw.SWATTN_VARIANT_MFMA
    assert sw.swattn_prefill_plan(desc(), 513, 188, check=False)[0] == -3
    # a 64-row chunk of GQA-4 rows spans at most 17 queries: 188 + 16 keys, one split
    p = sw.swattn_prefill_plan(desc(), 512, 188)
    assert p.num_splits == 1 and p.row_chunks == 32 and p.rows_per_chunk == 64 and p.workspace_bytes == 0
    # full-context prefill: ceil(min(4096, 4096 + 8) / 512) = 8 splits
    p = sw.swattn_prefill_plan(desc(), 512, 4096)
    assert p.num_splits == 8 and p.merge_grid > 0


def test_sixteen_row_chunks_only_while_the_grid_fits_the_cus():
    # the 16-row grid is B x Hkv x ceil(R / 16) x S workgroups; column splits by 2 or 4 where
    # it fits the CUs 2 or 4 times over.  Verify step: 96 16-row chunks, twice over 192
    p = sw.swattn_plan(desc(), 8, 188)
    assert p.rows_per_chunk == 16 and p.grid == 96 * 2
    # one layer (2 units): 4 16-row chunks, four column quarters each, one split per 64-key
    # tile of the chunk's 192 keys (3); with 4 splits forced, 16 chunk-splits, four quarters
    p = sw.swattn_plan(desc(batch=1), 8, 188)
    assert p.rows_per_chunk == 16 and p.num_splits == 3 and p.col_splits == 4 and p.grid == 4 * 4 * 3
    p = sw.swattn_plan(desc(batch=1, num_splits=4), 8, 188)
    assert p.rows_per_chunk == 16 and p.num_splits == 4 and p.grid == 16 * 4
    # plain decode: one 16-row chunk per KV head.  24 layers: 48, four times over 192;
    # 96 sequences: 192, no column split (before, 32-row chunks half of padding)
    p = sw.swattn_plan(desc(), 1, 188)
    assert p.rows_per_chunk == 16 and p.row_chunks == 1 and p.grid == 48 * 4
    p = sw.swattn_plan(desc(batch=96), 1, 188)
    assert p.rows_per_chunk == 16 and p.grid == 192
    # 96 units (48 problems): four times over is 384 > 256, twice over 192 -> 16-row chunks
    # without the column split; 160 units: 32-row chunks
    p = sw.swattn_plan(desc(batch=48), 8, 188)
    assert p.rows_per_chunk == 16 and p.grid == 48 * 2 * 2
    p = sw.swattn_plan(desc(batch=80), 8, 188)
    assert p.rows_per_chunk == 32 and p.grid == 80 * 2
    # 64 units: 16-row chunks again (256 workgroups)
    p = sw.swattn_plan(desc(batch=32), 8, 188)
    assert p.rows_per_chunk == 16 and p.grid == 256
    # full context (48 units x 4 or 8 splits) already fills the CUs: 32-row chunks
    assert sw.swattn_plan(desc(max_ctx_len=1024), 8, 4096).rows_per_chunk == 32
    assert sw.swattn_plan(desc(), 8, 4096).rows_per_chunk == 32
    # 64 queries: 64-row chunks; head_dim 128: 32-row chunks
    assert sw.swattn_plan(desc(), 64, 188).rows_per_chunk == 64
    assert sw.swattn_plan(desc(head_dim=128), 8, 188).rows_per_chunk == 32
    assert sw.swattn_plan(desc(head_dim=128), 64, 188).rows_per_chunk == 32
    # the batched workload (512 units) keeps 32-row chunks
    assert sw.swattn_plan(desc(batch=256), 8, 188).rows_per_chunk == 32


def test_small_launches_split_per_tile():
    # one layer of plain decode: 2 units, 191 keys -> one split per 64-key tile, whose
    # partials (4 rows x 256 x 4 splits x 4 B = 16 KiB) the last workgroup merges
    p = sw.swattn_plan(desc(batch=1), 1, 188)
    assert p.variant == sw.SWATTN_VARIANT_MFMA and p.num_splits == 3 and p.fused_merge == 1
    # one layer of the verify step: a 16-row chunk scans 188 + 4 keys -> 3 splits; a merge
    # group is a chunk's column quarter, 16 rows x 64 columns x 3 splits x 4 B = 12 KiB,
    # which its last workgroup merges
    p = sw.swattn_plan(desc(batch=1), 8, 188)
    assert p.variant == sw.SWATTN_VARIANT_MFMA and p.num_splits == 3 and p.fused_merge == 1
    assert p.col_splits == 4 and p.merge_grid == 0
    # head_dim 128 (no 16-row chunks): 32-row partials of 4 splits, 64 KiB -> no split
    p = sw.swattn_plan(desc(batch=1, head_dim=128), 8, 188)
    assert p.num_splits == 1 and p.rows_per_chunk == 32
    # 24 layers stacked: 48 units, no split
    assert sw.swattn_plan(desc(batch=24), 8, 188).num_splits == 1
    # head_dim 64 keeps 32-row chunks: 32 rows x 64 x 4 splits x 4 B = 32 KiB -> no split;
    # its plain decode (4 rows) splits, merged by the last workgroup
    assert sw.swattn_plan(desc(batch=1, head_dim=64), 8, 188).num_splits == 1
    p = sw.swattn_plan(desc(batch=1, head_dim=64), 1, 188)
    assert p.num_splits == 3 and p.fused_merge == 1
    # a forced split count still wins
    assert sw.swattn_plan(desc(batch=1, num_splits=4), 8, 188).num_splits == 4


def test_long_ranges_split_while_cus_idle():
    # 48 units, contexts of 1024 under a 4096 window: four splits of 256 keys
    # (192 workgroups on 256 CUs)
    assert sw.swattn_plan(desc(max_ctx_len=1024), 8, 4096).num_splits == 4
    # 4096 keys: the LDS table bound (8 splits) already fills the CUs
    assert sw.swattn_plan(desc(), 8, 4096).num_splits == 8
    # the verify window stays whole
    assert sw.swattn_plan(desc(), 8, 188).num_splits == 1


def test_verify_host_checks_return_before_launch():
    lib = sw.lib()
    d = desc(num_splits=2)
    plan = sw.swattn_plan(d, 8, 188)
    A = 1 << 20   # fake, aligned, never dereferenced: every call below fails on the host

    def call(q=A, k=2 * A, v=3 * A, bt=4 * A, ctx=5 * A, n_q=8, window=188, scale=0.0625,
             out=6 * A, ws=8 * A, wsb=None, dd=d):
        wsb = plan.workspace_bytes if wsb is None else wsb
        return sw.STATUS[lib.swattn_verify(ctypes.byref(dd), q, k, v, bt, ctx, n_q, window, scale,
                                           out, ws, wsb, None)]

    assert call(q=None) == "SWATTN_ERR_NULL"
    assert call(out=None) == "SWATTN_ERR_NULL"
    assert call(bt=None) == "SWATTN_ERR_NULL"
    assert call(q=A + 8) == "SWATTN_ERR_ALIGN"
    assert call(k=2 * A + 2) == "SWATTN_ERR_ALIGN"
    assert call(ctx=5 * A + 2) == "SWATTN_ERR_ALIGN"
    assert call(scale=float("nan")) == "SWATTN_ERR_ARG"
    assert call(scale=float("inf")) == "SWATTN_ERR_ARG"
    assert call(out=A + 16) == "SWATTN_ERR_ARG"                       # overlaps q
    assert call(ws=None) == "SWATTN_ERR_WORKSPACE"
    assert call(wsb=plan.workspace_bytes - 1) == "SWATTN_ERR_WORKSPACE"
    assert call(n_q=65) == "SWATTN_ERR_NQ"
    assert call(window=0) == "SWATTN_ERR_WINDOW"
    assert lib.swattn_check_inputs(ctypes.byref(d), None, 5 * A, 8, 188, None) == -1


def test_measurement_aids_host_checks_return_before_launch():
    # swattn_window_gather and swattn_stream_read refuse bad arguments on the host
    lib = sw.lib()
    d = desc()
    A = 1 << 20   # fake, aligned, never dereferenced: every call below fails on the host

    def gather(q=A, k=2 * A, v=3 * A, bt=4 * A, ctx=5 * A, n_q=8, window=188, parts=1, out=6 * A):
        return sw.STATUS[lib.swattn_window_gather(ctypes.byref(d), q, k, v, bt, ctx, n_q, window, parts, out, None)]

    assert gather(parts=0) == "SWATTN_ERR_ARG"
    assert gather(parts=17) == "SWATTN_ERR_ARG"
    assert gather(q=None) == "SWATTN_ERR_NULL"
    assert gather(out=None) == "SWATTN_ERR_NULL"
    assert gather(v=3 * A + 4) == "SWATTN_ERR_ALIGN"
    assert gather(n_q=65) == "SWATTN_ERR_NQ"
    assert gather(window=0) == "SWATTN_ERR_WINDOW"

    def read(src=A, nbytes=1 << 16, grid=512, xor_out=2 * A):
        return sw.STATUS[lib.swattn_stream_read(src, nbytes, grid, xor_out, None)]

    assert read(src=None) == "SWATTN_ERR_NULL"
    assert read(src=A + 8) == "SWATTN_ERR_ALIGN"
    assert read(xor_out=2 * A + 2) == "SWATTN_ERR_ALIGN"
    assert read(nbytes=24) == "SWATTN_ERR_ARG"
    assert read(nbytes=-16) == "SWATTN_ERR_ARG"
    assert read(grid=0) == "SWATTN_ERR_ARG"
    assert read(grid=65537) == "SWATTN_ERR_ARG"


def _longest_split(plan, n_q, G, window, ctx):
    """Most keys one workgroup scans under `plan` for a sequence of length ctx: the
    union of the windows of a row chunk's queries, in plan.num_splits near-equal parts
    (brute force over the chunks)."""
    R = n_q * G
    pos0 = ctx - n_q
    worst = 0
    for rc in range(plan.row_chunks):
        qs = [r // G for r in range(rc * plan.rows_per_chunk, min(R, (rc + 1) * plan.rows_per_chunk))]
        lo = max(0, pos0 + min(qs) - window + 1)
        hi = pos0 + max(qs) + 1
        worst = max(worst, -(-(hi - lo) // plan.num_splits))
    return worst


@pytest.mark.parametrize("kv", ["bf16", "e4m3", "f32"])
def test_every_split_fits_the_key_table(kv):
    # A workgroup keeps the source row of every key it scans in an LDS table of 512
    # entries (matrix-core kernel) or 256 (vector-ALU kernel); the plan must split long
    # ranges so that no workgroup scans more, whatever the launch size (single-sequence
    # full attention past 4096 keys included).
    kvd = {"bf16": sw.SWATTN_BF16, "e4m3": sw.SWATTN_FP8_E4M3, "f32": sw.SWATTN_F32}[kv]
    extra = dict(k_scale=16, v_scale=32) if kv == "e4m3" else {}
    checked = 0
    for D in (64, 128, 256):
        for H, Hkv in ((8, 2), (8, 8), (8, 1)):
            for batch in (1, 2, 8, 24, 200):
                for max_ctx in (300, 4096, 8192, 40000):
                    for n_q, window in ((1, 188), (8, 188), (1, 10 ** 6), (8, 10 ** 6), (64, 5000), (3, 2000)):
                        if n_q > max_ctx:
                            continue
                        d = desc(batch=batch, head_dim=D, num_heads=H, num_kv_heads=Hkv, kv_dtype=kvd,
                                 max_ctx_len=max_ctx, block_size=16, max_blocks_per_seq=-(-max_ctx // 16),
                                 **extra)
                        p = sw.swattn_plan(d, n_q, window)
                        table = 512 if p.variant == sw.SWATTN_VARIANT_MFMA else 256
                        worst = _longest_split(p, n_q, H // Hkv, window, max_ctx)
                        assert worst <= table, (D, H, Hkv, batch, max_ctx, n_q, window, p.as_dict(), worst)
                        checked += 1
    # the prefill entry point (n_q up to 512, 64-row chunks)
    for max_ctx, window in ((4096, 188), (8192, 10 ** 6), (40000, 4096)):
        d = desc(batch=1, kv_dtype=kvd, max_ctx_len=max_ctx, max_blocks_per_seq=-(-max_ctx // 16), **extra)
        p = sw.swattn_prefill_plan(d, 512, window)
        table = 512 if p.variant == sw.SWATTN_VARIANT_MFMA else 256
        assert _longest_split(p, 512, 4, window, max_ctx) <= table, p.as_dict()
        checked += 1
    assert checked > 500
