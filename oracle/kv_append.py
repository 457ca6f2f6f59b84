"""KV-cache append with bfloat16 rounding or E4M3 quantization (test
infrastructure only; see the package docstring for who may use it).

What it computes.  A verify step scores the target token and its 7 drafts
("The Fast Gemma Challenge: our verified-SOTA recipe, in full", manifest
SPECULATIVE_CONFIG), so the K and V rows of those n_new positions must already be
in the paged cache when attention runs; this is the write that puts them there.
For sequence b, new token i < n_new and KV head g, the row goes to position
t = ctx_len[b] - n_new + i (ctx_len counts the new tokens, as in the attention
call): block block_table[b][t // bs], offset t % bs.  A sequence whose ctx_len lies
outside [n_new, min(max_ctx_len, max_blocks * bs)], or a position whose block id
lies outside [0, num_blocks), is not written.

Element conversion (the pages fix no cache type; these are the library's rules):
* float32 -> bfloat16: round to nearest, ties to even, on the 16 dropped bits;
  NaN stays NaN (quiet) with its sign.
* bfloat16 -> float32: exact widening.
* float32 (or widened bfloat16) -> E4M3 with a per-head float32 scale s: the
  float32 quotient value / s (IEEE division, correctly rounded), then the nearest
  E4M3 value, ties to the even code; magnitudes above 448 (infinities included)
  saturate to 448; NaN gives the NaN code with the value's sign.  Stored code x
  scale is then the cache's value, as the attention call reads it.

Pinned in tests/test_kv_append_oracle.py: E4M3 rounding against torch's
float8_e4m3fn cast for every in-range input class (every code, every midpoint,
random values), saturation and NaN cases by hand, bfloat16 rounding against
torch's cast, and the write pattern against a dense reference built position by
position.
"""
import numpy as np

from .formats import e4m3_value_table

_E4M3 = e4m3_value_table()
_POS_CODES = np.arange(0x7F, dtype=np.uint8)          # 0x00 .. 0x7E: +0 .. 448
_POS_VALUES = _E4M3[:0x7F]                            # increasing, exact in float64


def quantize_e4m3(values, scale):
    """float32 array, float32 scale -> uint8 E4M3 codes (rules in the module doc)."""
    x = np.asarray(values, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        q = (x / np.float32(scale)).astype(np.float32)
    mag = np.abs(q.astype(np.float64))
    sign = np.signbit(q).astype(np.uint8) << 7
    out = np.empty(q.shape, dtype=np.uint8)
    nan = np.isnan(q)
    sat = ~nan & (mag >= 448.0)
    mid = ~nan & ~sat
    # nearest of the two neighbouring magnitudes; at an exact midpoint the even code
    m = mag[mid]
    hi = np.searchsorted(_POS_VALUES, m, side="left")          # first value >= m
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = m - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - m
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    exact = _POS_VALUES[hi] == m
    code = np.where(exact | pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    out[mid] = code
    out[sat] = 0x7E
    out[nan] = 0x7F
    return out | sign


def f32_to_bf16_rne(values):
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even."""
    x = np.asarray(values, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) & 0xFFFF
    quiet = ((bits >> 16) | 0x0040) & 0xFFFF                   # keep sign and payload top, set quiet bit
    return np.where(nan, quiet, rounded).astype(np.uint16)


def _to_f32(rows, new_format):
    if new_format == "f32":
        return np.asarray(rows, dtype=np.float32)
    if new_format == "bf16":
        return (np.asarray(rows, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(f"unknown input format {new_format!r}")


def convert_rows(rows, new_format, kv_format, scale=None):
    """New K or V rows [..., D] in new_format -> stored cache elements in kv_format."""
    if kv_format == "bf16" and new_format == "bf16":
        return np.asarray(rows, dtype=np.uint16).copy()
    x = _to_f32(rows, new_format)
    if kv_format == "f32":
        return x.copy()
    if kv_format == "bf16":
        return f32_to_bf16_rne(x)
    if kv_format == "e4m3":
        if scale is None:
            raise ValueError("E4M3 needs a scale")
        return quantize_e4m3(x, scale)
    raise ValueError(f"unknown cache format {kv_format!r}")


def append_kv(k_cache, v_cache, block_table, ctx_len, k_new, v_new, n_new, *, new_format, kv_format,
              k_scale=None, v_scale=None, max_ctx=None):
    """Return copies of (k_cache, v_cache) with the n_new rows of every sequence written.

    k_cache, v_cache: [num_blocks][Hkv][bs][D] in kv_format ("f32" float32, "bf16"
    uint16 bits, "e4m3" uint8 codes); k_new, v_new: [B][n_new][Hkv][D] in new_format
    ("f32" or "bf16"); k_scale, v_scale: [Hkv] float32 (E4M3 only).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    nb, Hkv, bs, D = kc.shape
    B = len(ctx_len)
    max_blocks = block_table.shape[1]
    limit = max_blocks * bs if max_ctx is None else min(max_ctx, max_blocks * bs)
    for b in range(B):
        ctx = int(ctx_len[b])
        if ctx < n_new or ctx > limit:
            continue
        for i in range(n_new):
            t = ctx - n_new + i
            phys = int(block_table[b, t // bs])
            if phys < 0 or phys >= nb:
                continue
            for g in range(Hkv):
                ks = None if k_scale is None else k_scale[g]
                vs = None if v_scale is None else v_scale[g]
                kc[phys, g, t % bs, :] = convert_rows(k_new[b, i, g], new_format, kv_format, ks)
                vc[phys, g, t % bs, :] = convert_rows(v_new[b, i, g], new_format, kv_format, vs)
    return kc, vc
