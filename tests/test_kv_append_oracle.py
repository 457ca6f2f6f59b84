"""CPU pins of oracle.kv_append: E4M3 quantization, bfloat16 rounding, write pattern.

The oracle's rounding is written from the format definitions; here it is checked
against torch's own casts (an independent implementation of the same formats),
against hand-derived cases, and against a dense reference of the write.
"""
import numpy as np
import pytest
import torch

from oracle import kv_append as ka
from oracle.formats import e4m3_value_table, decode_e4m3


TABLE = e4m3_value_table()
FINITE = [c for c in range(256) if not np.isnan(TABLE[c])]


def torch_e4m3(x32):
    return torch.from_numpy(np.asarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_every_code_round_trips():
    vals = TABLE[FINITE].astype(np.float32)
    got = ka.quantize_e4m3(vals, 1.0)
    assert np.array_equal(got, np.array(FINITE, dtype=np.uint8))


def test_midpoints_round_to_even_code():
    pos = np.array([c for c in range(0x7E)], dtype=np.int64)          # 0x00 .. 0x7D and their upper neighbour
    mids = ((TABLE[pos] + TABLE[pos + 1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (TABLE[pos] + TABLE[pos + 1]) / 2)   # exact in float32
    got = ka.quantize_e4m3(mids, 1.0)
    expect = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    assert np.array_equal(got, expect)
    assert np.array_equal(ka.quantize_e4m3(-mids, 1.0), expect | 0x80)
    assert np.array_equal(got, torch_e4m3(mids))


def test_matches_torch_cast_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.05, 1.0, 30.0, 200.0)]).astype(np.float32)
    x = x[np.abs(x) < 448.0]
    # just above and below every code
    vals = TABLE[FINITE].astype(np.float32)
    near = np.concatenate([np.nextafter(vals, np.float32(np.inf)), np.nextafter(vals, np.float32(-np.inf))])
    near = near[np.abs(near) < 448.0]
    x = np.concatenate([x, near]).astype(np.float32)
    assert np.array_equal(ka.quantize_e4m3(x, 1.0), torch_e4m3(x))


def test_saturation_nan_and_zero():
    x = np.array([448.0, 449.0, 463.9, 464.0, 1e30, np.inf, -448.0, -500.0, -np.inf, np.nan, -np.nan, 0.0, -0.0,
                  2.0 ** -10, 2.0 ** -10 * 3, 2.0 ** -11, 1e-30], dtype=np.float32)
    got = ka.quantize_e4m3(x, 1.0)
    assert list(got[:9]) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0xFE]
    assert got[9] == 0x7F and got[10] == 0xFF
    assert got[11] == 0x00 and got[12] == 0x80
    # 2^-10 is the midpoint of 0 and the smallest subnormal 2^-9: ties to the even code 0
    assert got[13] == 0x00
    # 3 * 2^-10 = 1.5 * 2^-9: midpoint of codes 1 and 2 -> 2
    assert got[14] == 0x02
    assert got[15] == 0x00 and got[16] == 0x00


def test_scale_divides_in_float32():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(5000).astype(np.float32) * 3
    for s in (np.float32(0.0123), np.float32(1.0), np.float32(7.5)):
        q = (x / s).astype(np.float32)
        assert np.array_equal(ka.quantize_e4m3(x, s), ka.quantize_e4m3(q, 1.0))
        back = decode_e4m3(ka.quantize_e4m3(x, s)) * np.float64(s)
        # in range, the stored value is within half an E4M3 step of the input
        inr = np.abs(q) < 448
        step = np.abs(back - x) / np.maximum(np.abs(x), 2 ** -6 * s)
        assert (step[inr] <= 2 ** -4 + 1e-12).all()


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(300000) * 10.0 ** rng.integers(-30, 30, 300000)).astype(np.float32)
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    ties = ((bits << 16) | 0x8000).view(np.float32)                   # exact halfway cases
    x = np.concatenate([x, ties[np.isfinite(ties)], np.array([np.inf, -np.inf, 0.0, -0.0], np.float32)])
    got = ka.f32_to_bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    nan = ka.f32_to_bf16_rne(np.array([np.nan, -np.nan], np.float32))
    assert ((nan & 0x7F80) == 0x7F80).all() and ((nan & 0x7F) != 0).all()
    assert (nan[0] >> 15) == 0 and (nan[1] >> 15) == 1


def dense_reference(k_cache, block_table, ctx_len, rows, n_new, conv):
    """The same write, done by walking positions of a dense per-sequence view."""
    out = np.array(k_cache, copy=True)
    nb, Hkv, bs, D = out.shape
    for b in range(len(ctx_len)):
        ctx = int(ctx_len[b])
        if ctx < n_new or ctx > block_table.shape[1] * bs:
            continue
        for pos in range(ctx - n_new, ctx):
            blk = block_table[b, pos // bs]
            if 0 <= blk < nb:
                out[blk, :, pos % bs, :] = conv(rows[b, pos - (ctx - n_new)])
    return out


@pytest.mark.parametrize("kv_format,new_format", [("bf16", "bf16"), ("bf16", "f32"), ("e4m3", "bf16"),
                                                  ("e4m3", "f32"), ("f32", "f32"), ("f32", "bf16")])
def test_write_pattern(kv_format, new_format):
    rng = np.random.default_rng(3)
    nb, Hkv, bs, D, B, n_new, max_blocks = 40, 2, 16, 32, 4, 8, 10
    dt = {"bf16": np.uint16, "e4m3": np.uint8, "f32": np.float32}[kv_format]
    if kv_format == "f32":
        kc = rng.standard_normal((nb, Hkv, bs, D)).astype(np.float32)
    else:
        kc = rng.integers(0, 0x7E if kv_format == "e4m3" else 0x4000, (nb, Hkv, bs, D)).astype(dt)
    vc = kc.copy()
    table = rng.permutation(nb)[:B * max_blocks].reshape(B, max_blocks).astype(np.int32)
    table[2, 1] = nb + 3                                  # a bad block id inside sequence 2's new rows
    ctx = np.array([8, 37, 25, 200], dtype=np.int32)      # sequence 3: ctx beyond max_blocks * bs, not written
    x = rng.standard_normal((B, n_new, Hkv, D)).astype(np.float32) * 2
    new = x if new_format == "f32" else ka.f32_to_bf16_rne(x)
    ks = np.array([0.01, 0.02], np.float32) if kv_format == "e4m3" else None
    k2, v2 = ka.append_kv(kc, vc, table, ctx, new, new, n_new,
                          new_format=new_format, kv_format=kv_format, k_scale=ks, v_scale=ks)
    for g in range(Hkv):
        ref = dense_reference(kc[:, g:g + 1], table, ctx, new[:, :, g:g + 1], n_new,
                              lambda r: ka.convert_rows(r[0], new_format, kv_format,
                                                        None if ks is None else ks[g]))
        assert np.array_equal(k2[:, g:g + 1], ref)
    # untouched rows stay as they were; sequence 3 writes nothing
    changed = np.argwhere((k2 != kc).any(axis=(1, 3)))
    written = set()
    for b in range(3):
        for pos in range(int(ctx[b]) - n_new, int(ctx[b])):
            blk = table[b, pos // bs]
            if 0 <= blk < nb:
                written.add((int(blk), pos % bs))
    assert set(map(tuple, changed.tolist())) <= written
