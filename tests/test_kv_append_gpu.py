"""GPU parity of swattn_append_kv (through the C ABI) against oracle.kv_append.

Byte-exact comparison of the whole cache after the call: the new rows converted
exactly as the oracle converts them, and nothing else touched (rows of a sequence
with a bad ctx_len and of a bad block id are left alone).
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_verify_kv_amd as sw
import synth
import gpu_util as gu

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TORCH = {"f32": torch.float32, "bf16": torch.int16, "e4m3": torch.uint8}
NP = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}
CODE = {"f32": sw.SWATTN_F32, "bf16": sw.SWATTN_BF16, "e4m3": sw.SWATTN_FP8_E4M3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sw.lib()


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def from_dev(t, fmt):
    a = t.cpu().numpy()
    return a.view(np.uint16) if fmt == "bf16" else a


def desc_for(B, Hkv, D, bs, max_blocks, nb, max_ctx, kv_format, ks, vs):
    d = sw.swattn_desc_t()
    d.batch, d.num_heads, d.num_kv_heads, d.head_dim = B, Hkv, Hkv, D
    d.block_size, d.max_blocks_per_seq, d.num_blocks, d.max_ctx_len = bs, max_blocks, nb, max_ctx
    d.q_dtype, d.kv_dtype, d.out_dtype = sw.SWATTN_BF16, CODE[kv_format], sw.SWATTN_BF16
    d.k_scale = None if ks is None else ks.data_ptr()
    d.v_scale = None if vs is None else vs.data_ptr()
    return d


def run_case(kv_format, new_format, B=5, Hkv=2, D=256, bs=16, n_new=8, nb=64, max_blocks=12, seed=0,
             specials=False):
    rng = np.random.default_rng(seed)
    gu.log(f"[append] kv {kv_format} new {new_format} B {B} Hkv {Hkv} D {D} bs {bs} n_new {n_new}")
    if kv_format == "f32":
        kc = rng.standard_normal((nb, Hkv, bs, D)).astype(np.float32)
    else:
        kc = rng.integers(0, 0x7E if kv_format == "e4m3" else 0x3F00, (nb, Hkv, bs, D)).astype(NP[kv_format])
    vc = np.flip(kc, axis=0).copy()
    table = rng.permutation(nb)[:B * max_blocks].reshape(B, max_blocks).astype(np.int32)
    ctx = rng.integers(n_new, max_blocks * bs + 1, B).astype(np.int32)
    ctx[1] = n_new                                          # the new rows are the whole sequence
    ctx[2] = n_new - 1 if n_new > 1 else 0                  # too short: not written
    bad_pos = int(ctx[3]) - 1
    table[3, bad_pos // bs] = -5                            # the last new row's block id is bad
    x = (rng.standard_normal((B, n_new, Hkv, D)) * rng.choice([1e-3, 0.3, 3.0, 60.0], (B, n_new, Hkv, 1)))
    x = x.astype(np.float32)
    if specials:
        flat = x.reshape(-1)
        flat[:8] = [np.nan, -np.inf, np.inf, 1e30, -1e30, 0.0, -0.0, 2.0 ** -140]
        if kv_format == "e4m3":
            # exact E4M3 midpoints once multiplied by the scale of head 0 (1.0)
            tab = oracle.e4m3_value_table()
            mids = ((tab[:0x7E] + tab[1:0x7F]) / 2).astype(np.float32)
            flat[8:8 + len(mids)] = mids
    y = -x[:, :, ::-1, :].copy() * 0.5
    if new_format == "bf16":
        xn, yn = oracle.f32_to_bf16_rne(x), oracle.f32_to_bf16_rne(y)
    else:
        xn, yn = x, y
    ks = vs = None
    kst = vst = None
    if kv_format == "e4m3":
        ks = np.array([1.0, 0.0137], np.float32)[:Hkv] if Hkv <= 2 else np.linspace(0.01, 1, Hkv).astype(np.float32)
        vs = (ks * 0.75).astype(np.float32)
        kst, vst = to_dev(ks), to_dev(vs)
    max_ctx = max_blocks * bs
    ek, ev = oracle.append_kv(kc, vc, table, ctx, xn, yn, n_new, new_format=new_format, kv_format=kv_format,
                              k_scale=ks, v_scale=vs, max_ctx=max_ctx)
    dk, dv = to_dev(kc), to_dev(vc)
    d = desc_for(B, Hkv, D, bs, max_blocks, nb, max_ctx, kv_format, kst, vst)
    sw.swattn_append_kv(d, to_dev(xn), to_dev(yn), CODE[new_format], to_dev(table), to_dev(ctx), n_new, dk, dv,
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    gk, gv = from_dev(dk, kv_format), from_dev(dv, kv_format)
    if specials and kv_format == "bf16" and new_format == "f32":
        # NaN payloads are the converter's choice: compare NaN-ness there, bits elsewhere
        for got, exp in ((gk, ek), (gv, ev)):
            gn = (got & 0x7F80) == 0x7F80
            gn &= (got & 0x7F) != 0
            en = ((exp & 0x7F80) == 0x7F80) & ((exp & 0x7F) != 0)
            assert np.array_equal(gn, en)
            assert np.array_equal(got[~gn], exp[~en])
        return
    assert np.array_equal(gk.view(np.uint8), np.ascontiguousarray(ek).view(np.uint8)), "K cache differs"
    assert np.array_equal(gv.view(np.uint8), np.ascontiguousarray(ev).view(np.uint8)), "V cache differs"


@pytest.mark.parametrize("kv_format,new_format", [("bf16", "bf16"), ("bf16", "f32"), ("e4m3", "bf16"),
                                                  ("e4m3", "f32"), ("f32", "f32"), ("f32", "bf16")])
def test_append_matches_oracle(kv_format, new_format):
    run_case(kv_format, new_format)


@pytest.mark.parametrize("kv_format,new_format", [("e4m3", "f32"), ("bf16", "f32"), ("e4m3", "bf16")])
def test_append_special_values(kv_format, new_format):
    run_case(kv_format, new_format, seed=1, specials=True)


def test_append_shapes():
    # (every case has >= 4 sequences: sequences 2 and 3 carry the bad ctx_len and block id)
    run_case("e4m3", "bf16", B=4, Hkv=1, D=64, bs=1, n_new=1, nb=128, max_blocks=30, seed=2)
    run_case("bf16", "f32", B=4, Hkv=4, D=128, bs=300, n_new=64, nb=8, max_blocks=2, seed=3)
    run_case("e4m3", "f32", B=4, Hkv=2, D=256, bs=16, n_new=512, nb=160, max_blocks=40, seed=4)


def test_append_then_verify_equals_cache_with_rows_present():
    # the verify workload's new rows, removed from the cache and appended back
    w, ref = gu.named("verify")
    t = gu.upload(w)
    bs, n_q = w.bs, w.n_q
    rows_k = np.zeros((w.B, n_q, w.Hkv, w.D), np.uint16)
    rows_v = np.zeros_like(rows_k)
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    for b in range(w.B):
        for i in range(n_q):
            pos = int(w.ctx_len[b]) - n_q + i
            blk, off = w.block_table[b, pos // bs], pos % bs
            rows_k[b, i], rows_v[b, i] = kc[blk, :, off], vc[blk, :, off]
            kc[blk, :, off] = 0x7FC0                      # NaN until the append writes them
            vc[blk, :, off] = 0x7FC0
    dk, dv = to_dev(kc).view(torch.bfloat16), to_dev(vc).view(torch.bfloat16)
    desc = sw.make_desc(t["q"], dk, t["bt"], int(w.ctx_len.max()))
    sw.swattn_append_kv(desc, to_dev(rows_k), to_dev(rows_v), sw.SWATTN_BF16, t["bt"], t["ctx"], n_q, dk, dv,
                        torch.cuda.current_stream().cuda_stream)
    out, _ = sw.verify(t["q"], dk, dv, t["bt"], t["ctx"], n_q, w.window, w.scale, int(w.ctx_len.max()),
                       out_dtype=sw.SWATTN_F32)
    torch.cuda.synchronize()
    gu.check(out.cpu().numpy().astype(np.float64), ref, w.kv_dtype, True, label="append+verify")


def test_append_host_errors():
    d = desc_for(1, 2, 256, 16, 4, 8, 64, "e4m3", None, None)
    x = torch.zeros((1, 8, 2, 256), dtype=torch.int16, device=DEV)
    c = torch.zeros((8, 2, 16, 256), dtype=torch.uint8, device=DEV)
    tb = torch.zeros((1, 4), dtype=torch.int32, device=DEV)
    cl = torch.full((1,), 8, dtype=torch.int32, device=DEV)
    st = sw.swattn_append_kv(d, x, x, sw.SWATTN_BF16, tb, cl, 8, c, c, check=False)
    assert sw.STATUS[st] == "SWATTN_ERR_DTYPE"                  # E4M3 without scales
    d = desc_for(1, 2, 256, 16, 4, 8, 64, "bf16", None, None)
    assert sw.STATUS[sw.swattn_append_kv(d, x, x, sw.SWATTN_BF16, tb, cl, 0, c, c, check=False)] == "SWATTN_ERR_NQ"
    assert sw.STATUS[sw.swattn_append_kv(d, x, x, sw.SWATTN_FP8_E4M3, tb, cl, 8, c, c, check=False)] == "SWATTN_ERR_DTYPE"
