"""Seeded synthetic verify-step inputs.

Recipe (the pages' workload is a private prompt set that is not available; these
inputs stand in for the KV state of one stream with up to 4096 positions):

* draws come from ``numpy.random.default_rng(seed)`` in a fixed order:
  context lengths (when drawn), block permutation, Q, K, V, then the set of Q
  rows scaled by ``hot_scale`` (when ``hot_frac`` > 0);
* values are float32 N(0, 1), rounded to bfloat16 with round-to-nearest-even
  (torch's conversion) when the storage type is bf16, or quantised to OCP E4M3
  with one scale per KV head (``amax / 448`` over that head's drawn values,
  round-to-nearest-even, saturating) when it is e4m3;
* only the ``recent`` most recent positions of each sequence get random values;
  older positions inside the sequence hold finite sentinels (K = +4, V = 100) and
  positions at or beyond ``ctx_len`` inside a referenced block hold NaN, so that a
  kernel that leaks weight outside the window, or reads past the context, shows;
* the physical block pool is the blocks the sequences reference, in a random
  permutation, plus ``extra_blocks`` blocks that no table references, filled
  with NaN (so that a read outside the referenced blocks shows); unused
  block-table entries are -1.
"""
from dataclasses import dataclass, field
import math

import numpy as np
import torch

F32, BF16, E4M3 = "f32", "bf16", "e4m3"
_K_SENTINEL = 4.0
_V_SENTINEL = 100.0
_E4M3_MAX = 448.0
_E4M3_NAN = 0x7F
_BF16_NAN = 0x7FC0


def to_bf16_bits(x):
    """float32 array -> uint16 bfloat16 bit patterns (round-to-nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def quantize_e4m3(x, scale):
    """float32 array / scale -> uint8 OCP E4M3 codes (RNE, saturating at 448)."""
    y = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)) / float(scale)
    y = y.clamp(-_E4M3_MAX, _E4M3_MAX).to(torch.float8_e4m3fn)
    return y.view(torch.uint8).numpy()


@dataclass
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    D: int
    n_q: int
    window: int
    scale: float
    bs: int
    q_dtype: str
    kv_dtype: str
    q: np.ndarray              # [B, n_q, H, D] float32, or uint16 bf16 bits
    k_cache: np.ndarray        # [num_blocks, Hkv, bs, D] float32 / uint16 / uint8
    v_cache: np.ndarray
    block_table: np.ndarray    # [B, max_blocks] int32
    ctx_len: np.ndarray        # [B] int32
    k_scale: np.ndarray = None  # [Hkv] float32 (e4m3 only)
    v_scale: np.ndarray = None
    meta: dict = field(default_factory=dict)

    @property
    def num_blocks(self):
        return self.k_cache.shape[0]

    @property
    def max_blocks(self):
        return self.block_table.shape[1]

    @property
    def q_format(self):
        return {F32: "float", BF16: "bf16"}[self.q_dtype]

    @property
    def kv_format(self):
        return {F32: "float", BF16: "bf16", E4M3: "e4m3"}[self.kv_dtype]


def make_workload(name, *, B, H, Hkv, D, n_q, window, ctx, bs, seed,
                  q_dtype=BF16, kv_dtype=BF16, scale=None, recent=None,
                  shuffle=True, hot_frac=0.0, hot_scale=8.0, max_blocks=None,
                  ctx_range=None, extra_blocks=0):
    """Build one seeded workload.

    ctx: an int (same context for every sequence) or a sequence of ints; ignored
    when ``ctx_range=(lo, hi)`` is given, in which case each context length is
    drawn uniformly from the integers lo..hi inclusive.
    recent: how many of the most recent positions of each sequence hold random
    values (default: all of them).
    extra_blocks: physical blocks added to the pool that no sequence references;
    they hold NaN.  The table's blocks are the first ones of a permutation of the
    whole pool (with 0 extra blocks the draws are those of the plain pool).
    """
    rng = np.random.default_rng(seed)
    if ctx_range is not None:
        ctx_len = rng.integers(ctx_range[0], ctx_range[1] + 1, size=B).astype(np.int64)
    else:
        ctx_len = np.broadcast_to(np.asarray(ctx, dtype=np.int64), (B,)).copy()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nblk = [(int(c) + bs - 1) // bs for c in ctx_len]
    if max_blocks is None:
        max_blocks = max(nblk)
    used = int(sum(nblk))
    pool = used + int(extra_blocks)
    perm = rng.permutation(pool) if shuffle else np.arange(pool)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    start = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[start:start + nblk[b]]
        start += nblk[b]

    q = rng.standard_normal((B, n_q, H, D), dtype=np.float32)

    # K then V: random values for the recent positions, sentinels before them,
    # NaN after the context inside the last referenced block.
    draws = []
    for _ in range(2):
        per_seq = []
        for b in range(B):
            c = int(ctx_len[b])
            r0 = 0 if recent is None else max(0, c - recent)
            pos = np.arange(c)
            phys = table[b, pos // bs].astype(np.int64)
            off = pos % bs
            vals = rng.standard_normal((c - r0, Hkv, D), dtype=np.float32)
            per_seq.append((phys[:r0], off[:r0], phys[r0:], off[r0:], vals))
        draws.append(per_seq)

    if hot_frac > 0.0:
        rows = B * n_q * H
        n_hot = int(round(hot_frac * rows))
        hot = rng.choice(rows, size=n_hot, replace=False)
        qf = q.reshape(rows, D)
        qf[hot] *= hot_scale
        q = qf.reshape(B, n_q, H, D)

    if q_dtype == BF16:
        q_store = to_bf16_bits(q)
    elif q_dtype == F32:
        q_store = q
    else:
        raise ValueError(f"unsupported q dtype {q_dtype}")

    shape = (pool, Hkv, bs, D)
    stores, scales = [], []
    for per_seq, sentinel in zip(draws, (_K_SENTINEL, _V_SENTINEL)):
        if kv_dtype == F32:
            store = np.full(shape, np.nan, dtype=np.float32)
            fill, conv, sc = np.float32(sentinel), (lambda x, g=None: x), None
        elif kv_dtype == BF16:
            store = np.full(shape, _BF16_NAN, dtype=np.uint16)
            fill, conv, sc = to_bf16_bits(np.float32([sentinel]))[0], (lambda x, g=None: to_bf16_bits(x)), None
        elif kv_dtype == E4M3:
            # One scale per KV head from that head's drawn values; sentinels saturate.
            amax = np.zeros(Hkv, dtype=np.float32)
            for (_, _, _, _, vals) in per_seq:
                if vals.size:
                    amax = np.maximum(amax, np.abs(vals).max(axis=(0, 2)))
            sc = np.where(amax > 0, amax / _E4M3_MAX, 1.0).astype(np.float32)
            store = np.full(shape, _E4M3_NAN, dtype=np.uint8)
            fill = None
            conv = None
        else:
            raise ValueError(f"unsupported kv dtype {kv_dtype}")
        for (ps, os_, pr, or_, vals) in per_seq:
            if kv_dtype == E4M3:
                for g in range(Hkv):
                    store[ps, g, os_, :] = quantize_e4m3(np.float32([sentinel]), sc[g])[0]
                    store[pr, g, or_, :] = quantize_e4m3(vals[:, g, :], sc[g])
            else:
                store[ps, :, os_, :] = fill
                store[pr, :, or_, :] = conv(vals)
        stores.append(store)
        scales.append(sc)
    k_store, v_store = stores
    k_scale, v_scale = scales

    return Workload(name=name, B=B, H=H, Hkv=Hkv, D=D, n_q=n_q, window=window,
                    scale=float(scale), bs=bs, q_dtype=q_dtype, kv_dtype=kv_dtype,
                    q=q_store, k_cache=k_store, v_cache=v_store,
                    block_table=table, ctx_len=ctx_len.astype(np.int32),
                    k_scale=k_scale, v_scale=v_scale,
                    meta=dict(seed=seed, recent=recent, shuffle=shuffle, extra_blocks=int(extra_blocks)))


def _c0(**kw):
    return make_workload("tiny_decode_fp32_d64_ctx300", B=1, H=2, Hkv=1, D=64, n_q=1,
                         window=188, ctx=300, bs=300, seed=0, q_dtype=F32,
                         kv_dtype=F32, scale=1.0 / 8.0, recent=188, shuffle=False, **kw)


def _c1(window=188, **kw):
    return make_workload(f"verify_24layers_h8kv2_d256_bf16_ctx4096_w{window}_nq8", B=24, H=8,
                         Hkv=2, D=256, n_q=8, window=window, ctx=4096, bs=16, seed=1,
                         recent=window + 8 - 1, **kw)


def _decode(window=188, **kw):
    return make_workload(f"decode_24layers_h8kv2_d256_bf16_ctx4096_w{window}_nq1", B=24, H=8,
                         Hkv=2, D=256, n_q=1, window=window, ctx=4096, bs=16, seed=6,
                         recent=window, **kw)


def _c2(ctx, **kw):
    return make_workload(f"fullctx_24layers_h8kv2_d256_bf16_ctx{ctx}_w4096_nq8", B=24,
                         H=8, Hkv=2, D=256, n_q=8, window=4096, ctx=ctx, bs=16, seed=2, **kw)


def _c3(window=188, **kw):
    return make_workload(f"wideverify_24layers_h8kv2_d256_bf16_ctx4096_w{window}_nq64", B=24,
                         H=8, Hkv=2, D=256, n_q=64, window=window, ctx=4096, bs=16, seed=3,
                         recent=window + 64 - 1, hot_frac=614 / 12288, **kw)


def _c4(kv_dtype, window=188, **kw):
    return make_workload(f"batched_256seq_h8kv2_d256_{kv_dtype}kv_ctxU188-4096_w{window}_nq8",
                         B=256, H=8, Hkv=2, D=256, n_q=8, window=window, ctx=None, bs=16,
                         seed=4, kv_dtype=kv_dtype, recent=window + 8 - 1,
                         ctx_range=(188, 4096), max_blocks=256, **kw)


def _prefill(n_q, window=188, **kw):
    return make_workload(f"prefill_24layers_h8kv2_d256_bf16_ctx4096_w{window}_nq{n_q}", B=24, H=8,
                         Hkv=2, D=256, n_q=n_q, window=window, ctx=4096, bs=16, seed=5,
                         recent=window + n_q - 1, **kw)


# The five workloads of the build: tiny decode, single-stream verify, the
# full-context split-KV contrast (three lengths), wide verify and the batched
# stress test (fp8 and bf16 KV); then chunked prefill and single-stream plain
# decode (the verify workload with one query per step).
NAMED = {
    "tiny_decode": _c0,
    "verify": _c1,
    "fullctx_1024": lambda **kw: _c2(1024, **kw),
    "fullctx_2048": lambda **kw: _c2(2048, **kw),
    "fullctx_4096": lambda **kw: _c2(4096, **kw),
    "wide_verify": _c3,
    "batched_fp8": lambda **kw: _c4(E4M3, **kw),
    "batched_bf16": lambda **kw: _c4(BF16, **kw),
    "prefill_512": lambda **kw: _prefill(512, **kw),
    "decode": _decode,
}


def named_workload(key, **overrides):
    """A named workload; keyword overrides go to make_workload (e.g. extra_blocks)."""
    return NAMED[key](**overrides)

